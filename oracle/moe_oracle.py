"""float64 reference of the null-expert MoE layer forward (test infrastructure).

Notation follows [Review] section 3: N real experts E_1..E_N, a null expert
whose output is zero, the null logit duplicated M times before top-K, a shared
expert, routing weights renormalised over the chosen real experts only.
Pool ids: 0..N-1 are the real experts, N..N+M-1 are the M null copies.

Readings where the pages leave a step open (each is listed in the design notes):
  * the null logit is router row N plus a scalar bias b plus an optional
    per-token bias b_t; the real logits carry no bias;
  * a real expert must be strictly larger than the null logit to beat it (the
    threshold paragraph says the chosen reals exceed the null logit), so at an
    exact tie the null copy wins; equal reals are ordered by lower index, null
    copies by lower copy id;
  * the K slots of a token list its chosen reals first, by (logit desc, index
    asc), then the null copies N, N+1, ... in copy-id order;
  * with M = 0 the null row is ignored and the pool is the N reals (plain top-K);
  * the expert FFN is SwiGLU without biases: W_down (silu(W_gate a) * W_up a);
  * zero-compute variants ([Review] "why null rather than copy experts" table and
    the [MoE++] zero / copy / constant experts): a null slot outputs 0 (null),
    the token x (copy) or a vector v (constant). For copy and constant slots the
    gate weights are a softmax over all K chosen pool entries, null slots taking
    the null logit, since a renormalisation over the reals alone would give the
    null slots weight 0 and the layer could not become (1 - rho) x + rho y_dense
    in expectation as the table says.
"""
import numpy as np

from workloads import bf16_bits_to_f32

f64 = np.float64


def _vals(a):
    """Exact float64 values of a stored tensor (bf16 bit patterns or floats)."""
    a = np.asarray(a)
    return bf16_bits_to_f32(a).astype(f64) if a.dtype == np.uint16 else a.astype(f64)


# ---------------------------------------------------------------- router
def router_logits(x, w_router, null_bias=0.0, null_bias_tok=None):
    """Router scores s = x W_g^T over N+1 rows; column N is the effective null
    logit s_N + b (+ b_t).  [Review] "Null Expert mechanism": the router is
    widened to N+1 logits, the last one belonging to the null expert; [Primer]
    section 3: the router is a bias-free linear map of the token state."""
    x = np.asarray(x, dtype=f64)
    w = np.asarray(w_router, dtype=f64)
    s = x @ w.T
    s[:, -1] += f64(null_bias)
    if null_bias_tok is not None:
        s[:, -1] += np.asarray(null_bias_tok, dtype=f64)
    return s


# ---------------------------------------------------------------- selection
def _pool(logits, N, M):
    """Extended pool [s_1..s_N, s_null x M] ([Review] "Null Expert mechanism")."""
    s = np.asarray(logits, dtype=f64)
    T = s.shape[0]
    v = np.empty((T, N + M), dtype=f64)
    v[:, :N] = s[:, :N]
    if M:
        v[:, N:] = s[:, N:N + 1]
    return v


def select(logits, N, M, K):
    """Top-K over the pool under the total order
         larger value first; at equal value a null copy before a real expert;
         then lower real index; then lower null copy id,
    i.e. the threshold rule of [Review] "threshold interpretation": a real
    expert is chosen over a null copy only if its logit is strictly larger.
    Returns (topk_idx [T,K] int32, n_real [T] int32): the chosen reals in
    (value desc, index asc) order, followed by the chosen null copy ids."""
    T = logits.shape[0]
    v = _pool(logits, N, M)
    ids = np.broadcast_to(np.arange(N + M), v.shape)
    is_real = ids < N
    # np.lexsort sorts by the last key first: value desc, then null first, then id.
    order = np.lexsort((ids, is_real, -v), axis=-1)[:, :K]
    chosen_real = order < N
    n_real = chosen_real.sum(axis=1).astype(np.int32)
    topk = np.empty((T, K), dtype=np.int32)
    for t in range(T):
        reals = order[t][chosen_real[t]]          # already in (value desc, index asc) order
        nulls = np.sort(order[t][~chosen_real[t]])
        topk[t] = np.concatenate([reals, nulls])
    return topk, n_real


def decisive_gap(logits, N, M, K):
    """Smallest |v_a - v_b| between a chosen and an unchosen pool entry; a
    routing difference between two implementations at a token is admissible
    only where this gap is below the flip tolerance. Where the nearest chosen and
    unchosen entries are the same infinity (a +inf null logit: its copies are both
    chosen and left over), no finite change of a logit moves the decision, which the
    tie rule settles: the gap is taken as infinite."""
    v = _pool(logits, N, M)
    P = N + M
    if K >= P:
        return np.full(v.shape[0], np.inf)
    topk, _ = select(logits, N, M, K)
    T = v.shape[0]
    chosen = np.zeros((T, P), dtype=bool)
    np.put_along_axis(chosen, topk.astype(np.int64), True, axis=1)
    lo = np.where(chosen, v, np.inf).min(axis=1)
    hi = np.where(~chosen, v, -np.inf).max(axis=1)
    same_inf = np.isinf(lo) & (lo == hi)
    gap = np.abs(np.where(same_inf, 0.0, lo) - np.where(same_inf, 0.0, hi))
    return np.where(same_inf, np.inf, gap)


def renorm_weights(logits, topk_idx, N):
    """Weights renormalised over the chosen real experts only ([Review] "Null
    Expert mechanism"; the same as the pool softmax restricted to the chosen
    reals and rescaled to sum 1, and as the [MoE++] gating sequence). Computed
    as a softmax over the chosen real logits, max-shifted. Null slots get 0;
    a token with no real expert gets all zeros."""
    s = np.asarray(logits, dtype=f64)
    T, K = topk_idx.shape
    w = np.zeros((T, K), dtype=f64)
    for t in range(T):
        sel = [k for k in range(K) if topk_idx[t, k] < N]
        if not sel:
            continue
        vals = s[t, topk_idx[t, sel]]
        e = np.exp(vals - vals.max())
        w[t, sel] = e / e.sum()
    return w


def chosen_weights(logits, topk_idx, N):
    """Weights of the copy / constant variants: a softmax over all K chosen pool
    entries, null slots taking the effective null logit (column N), max-shifted.
    An entry equal to the maximum has numerator 1, which for a null logit at +inf
    is the limit (every chosen null copy equally, the reals 0)."""
    s = np.asarray(logits, dtype=f64)
    T, K = topk_idx.shape
    if not K:
        return np.zeros((T, 0))
    vals = np.where(topk_idx < N, np.take_along_axis(s, np.minimum(topk_idx, N), axis=1), s[:, N:N + 1])
    mx = vals.max(axis=1, keepdims=True)
    with np.errstate(invalid="ignore"):
        e = np.where(vals == mx, 1.0, np.exp(vals - mx))
    return e / e.sum(axis=1, keepdims=True)


def route(logits, N, M, K, null_kind="zero"):
    topk, n_real = select(logits, N, M, K)
    w = renorm_weights(logits, topk, N) if null_kind == "zero" else chosen_weights(logits, topk, N)
    return topk, w, n_real


def null_source(wl, rows=None):
    """Rows that a null slot adds (times its weight): None for null experts, the
    tokens x for copy experts, the vector v (broadcast) for constant experts."""
    kind = wl.cfg.null_kind
    if kind == "zero":
        return None
    if kind == "copy":
        x = wl.values("x")
        return x if rows is None else x[rows]
    if kind == "constant":
        return wl.values("null_value")
    raise ValueError(kind)


# ---------------------------------------------------------------- dispatch
def permute(topk_idx, N):
    """Stable argsort of the flat slot ids (token-major, then slot) by expert id
    with every null id (>= N) sorted past the end and cut off ([Review]
    "implementation": argsort sends indices >= N to the end and the list is
    truncated before the grouped GEMM).
    Returns counts [N], offsets [N+1], perm_token [R], slot_pos [T,K] (-1 = null)."""
    T, K = topk_idx.shape
    flat = topk_idx.reshape(-1).astype(np.int64)
    key = np.where((flat >= 0) & (flat < N), flat, N)
    order = np.argsort(key, kind="stable")
    R = int((key < N).sum())
    perm_flat = order[:R]
    counts = np.bincount(key[key < N], minlength=N).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    slot_pos = np.full(T * K, -1, dtype=np.int32)
    slot_pos[perm_flat] = np.arange(R, dtype=np.int32)
    perm_token = (perm_flat // K).astype(np.int32)
    return counts, offsets, perm_token, slot_pos.reshape(T, K)


# ---------------------------------------------------------------- experts
def silu(z):
    z = np.asarray(z, dtype=f64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_ffn(a, w_gate, w_up, w_down):
    """One expert applied to the rows of a: W_down (silu(W_gate a) * (W_up a)).
    Each row depends only on itself ([Primer] section 2: the FFN is per-token),
    which is what makes permute -> grouped GEMM -> combine exact."""
    a = np.asarray(a, dtype=f64)
    h = silu(a @ _vals(w_gate).T) * (a @ _vals(w_up).T)
    return h @ _vals(w_down).T


def expert_ffn_grouped(a, offsets, w_gate, w_up, w_down):
    """Per segment e (rows offsets[e]..offsets[e+1]) apply expert e: the role of
    the grouped GEMM in [Review] "implementation"."""
    a = np.asarray(a, dtype=f64)
    out = np.zeros((a.shape[0], np.shape(w_down)[1]), dtype=f64)
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            out[lo:hi] = swiglu_ffn(a[lo:hi], w_gate[e], w_up[e], w_down[e])
    return out


def combine(y_perm, slot_pos, topk_w, y_shared=None, d_model=None, null_src=None):
    """y_t = E_shared(x_t) + sum_k w_tk E_{i_k}(x_t), summed in slot order
    ([Review] core formula of the token-choice layer with a shared expert); a
    null slot adds E_null = 0, or with ``null_src`` w_tk times its row t ([T, d],
    copy experts) or the one vector ([d], constant experts)."""
    T, K = slot_pos.shape
    d = y_perm.shape[1] if d_model is None else d_model
    y = np.zeros((T, d), dtype=f64) if y_shared is None else np.array(y_shared, dtype=f64)
    src = None if null_src is None else np.asarray(null_src, dtype=f64)
    for k in range(K):
        p = slot_pos[:, k]
        m = p >= 0
        y[m] += topk_w[m, k][:, None] * np.asarray(y_perm, f64)[p[m]]
        if src is not None:
            n = ~m
            y[n] += topk_w[n, k][:, None] * (src[n] if src.ndim == 2 else src[None, :])
    return y


# ---------------------------------------------------------------- statistics
def pool_softmax(logits, N, M):
    """Pool softmax p_t over [s_1..s_N, s_null x M] and lse_t = log sum_i e^{v_t,i},
    max-shifted ([Review] load-balance loss and z-loss). A null logit of +inf (an
    infinite per-token null bias, M > 0) takes the limit of a growing null logit:
    each null copy 1/M, every real 0, and lse_t = +inf. Returns (p [T, N+M], lse [T])."""
    v = _pool(logits, N, M)
    T, P = v.shape
    inf_null = np.zeros(T, dtype=bool) if M == 0 else np.isposinf(v[:, N])
    if inf_null.any():
        # the limit: the null copies at 0 and the reals at -inf after the shift
        limit = np.where(np.arange(P) >= N, 0.0, -np.inf)
        v = np.where(inf_null[:, None], limit[None, :], v)
    m = v.max(axis=1, keepdims=True) if P else np.zeros((T, 1))
    ex = np.exp(v - m)
    z = ex.sum(axis=1, keepdims=True)
    p = ex / z
    lse = np.where(inf_null, np.inf, (m + np.log(z))[:, 0])
    return p, lse


def aux_stats(logits, topk_idx, N, M, K):
    """Load-balance and z-loss statistics over the N+M pool.
      p_t = softmax of the pool [s_1..s_N, s_null x M]      ([Review] load-balance loss)
      P_i = mean_t p_t,i ; counts_i = #slots routed to pool id i ; f_i = counts_i / T
      L_bal = N * sum_{i<N+M} f_i P_i                          ([Review] load-balance loss)
      L_z = mean_t (log sum_{i<N+M} exp v_t,i)^2              ([Review] z-loss; [Primer] 4.3)
    plus mean_r = mean number of chosen reals per token ([Review] expected
    active experts; r/K is the compute intensity of [Summary] Figure 4).
    A token whose null logit is +inf contributes the limit of ``pool_softmax``
    (1/M per null copy) to P and lse = +inf, so L_z = +inf."""
    p, lse = pool_softmax(logits, N, M)
    T, P = p.shape
    Pm = p.mean(axis=0) if T else np.zeros(P)
    flat = topk_idx.reshape(-1)
    counts = np.bincount(flat[(flat >= 0) & (flat < P)], minlength=P).astype(np.int64)
    f = counts / T if T else np.zeros(P)
    L_bal = N * float((f * Pm).sum())
    L_z = float((lse ** 2).mean()) if T else 0.0
    n_real = (topk_idx < N).sum(axis=1)
    mean_r = float(n_real.mean()) if T else 0.0
    return dict(f=f, P=Pm, counts=counts, L_bal=L_bal, L_z=L_z, mean_r=mean_r, lse=lse)


# ---------------------------------------------------------------- layer
def layer_forward(wl, logits=None, K=None, M=None):
    """Whole layer on a ``workloads.Workload``. ``logits`` (T x (N+1), column N
    effective) replaces the router GEMM when given, e.g. the GPU's fp32 logits
    for routing-parity checks."""
    cfg = wl.cfg
    N = cfg.n_experts
    M = cfg.n_null if M is None else M
    K = cfg.top_k if K is None else K
    x = wl.values("x")
    if logits is None:
        logits = router_logits(x, wl.values("w_router"), wl.null_bias, wl.null_bias_tok)
    logits = np.asarray(logits, dtype=f64)
    topk, w, n_real = route(logits, N, M, K, cfg.null_kind)
    counts, offsets, perm_token, slot_pos = permute(topk, N)
    xp = x[perm_token]
    yp = expert_ffn_grouped(xp, offsets, wl.w_gate, wl.w_up, wl.w_down)
    ys = None
    if cfg.d_ff_shared:
        ys = swiglu_ffn(x, wl.ws_gate, wl.ws_up, wl.ws_down)
    y = combine(yp, slot_pos, w, ys, d_model=cfg.d_model, null_src=null_source(wl))
    aux = aux_stats(logits, topk, N, M, K)
    return dict(logits=logits, topk_idx=topk, topk_w=w, n_real=n_real, counts=counts,
                offsets=offsets, perm_token=perm_token, slot_pos=slot_pos, x_perm=xp,
                y_perm=yp, y_shared=ys, y=y, aux=aux)


def layer_dense(wl, logits=None, K=None, M=None, tokens=None):
    """The same layer written densely: with G the T x N matrix of routing weights
    (G[t,e] = weight of e if chosen, else 0), y = E_shared(x) + sum_e G[:,e] E_e(x)
    ([Review] core formula; the routing matrix of [Review] section 2). Each
    expert is applied to every token, no permutation is involved. ``tokens``
    restricts the rows evaluated (sampled checks at large sizes). Only tokens
    with G[t,e] != 0 are passed through expert e, which changes nothing since
    the other terms are multiplied by zero."""
    cfg = wl.cfg
    N = cfg.n_experts
    M = cfg.n_null if M is None else M
    K = cfg.top_k if K is None else K
    x = wl.values("x")
    rows = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    xs = x[rows]
    if logits is None:
        btok = None if wl.null_bias_tok is None else wl.null_bias_tok[rows]
        logits = router_logits(xs, wl.values("w_router"), wl.null_bias, btok)
    else:
        logits = np.asarray(logits, dtype=f64)[rows]
    topk, w, _ = route(logits, N, M, K, cfg.null_kind)
    G = np.zeros((len(rows), N), dtype=f64)
    for k in range(K):
        real = topk[:, k] < N
        G[np.nonzero(real)[0], topk[real, k]] += w[real, k]
    y = np.zeros((len(rows), cfg.d_model), dtype=f64)
    if cfg.d_ff_shared:
        y += swiglu_ffn(xs, wl.ws_gate, wl.ws_up, wl.ws_down)
    src = null_source(wl, rows)
    if src is not None:
        g_null = (w * (topk >= N)).sum(axis=1)  # total weight of the null slots
        y += g_null[:, None] * (src if src.ndim == 2 else src[None, :])
    for e in range(N):
        used = G[:, e] != 0
        if used.any():
            y[used] += G[used, e][:, None] * swiglu_ffn(xs[used], wl.w_gate[e], wl.w_up[e], wl.w_down[e])
    return y, topk, w
