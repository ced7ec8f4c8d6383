"""float64 reference of the null-expert MoE layer backward pass (test infrastructure).

The training objective this differentiates is

    L = <dy, y> + alpha * L_bal + beta * L_z

for an upstream gradient dy of the layer output y and the two auxiliary losses of
[Review] section 3 ("load-balance loss", "z-loss"; [Primer] sections 4.2 and 4.3),
with the coefficients passed in (the pages train with 2e-2 and 1e-3). Everything is
the chain rule through the forward of ``moe_oracle.layer_forward`` with the routing
decision held fixed (top-K is piecewise constant in the logits, so it has no
derivative; the counts f_i are constants for the same reason):

  combine      y_t = ys_t + sum_{k real} g_tk Y_{p(t,k)}
               dY_p = g_tk dy_t,                 dg_tk = <dy_t, Y_p>
  weights      g_t = softmax over the chosen reals S_t of s_t (renormalised)
               ds_tj = g_tj (dg_tj - sum_{i in S_t} g_ti dg_ti)   for j in S_t
  L_bal        = N sum_i f_i P_i,  P_i = mean_t p_ti,  p_t = softmax of the pool
               [s_t,1..N, s_null x M]; d/dv_tc = (N/T) p_tc (f_c - sum_i f_i p_ti)
  L_z          = mean_t lse_t^2;   d/dv_tc = (2/T) lse_t p_tc
               the M null copies all read the null logit, so its gradient is the
               sum over the copies (and 0 when M = 0: the null row is not used)
  null at +inf a token whose null logit is +inf (infinite per-token bias) has the
               limit pool softmax (1/M per null copy, reals 0) and lse = +inf, so
               L_z = +inf and its z-loss gradient has no finite value: it is taken
               as 0. Its balance term is 0 as well (p is constant in every finite
               logit), so the token's logit gradient is the weight term alone.
  router       s = x W_r^T (+ constant null biases): dW_r = ds^T x, dx += ds W_r
  expert e     g = a W_g^T, u = a W_u^T, h = silu(g) u, Y = h W_d^T:
               dh = dY W_d, dW_d = dY^T h, dg = dh u silu'(g), du = dh silu(g),
               silu'(z) = sigma(z) (1 + z (1 - sigma(z))),
               dW_g = dg^T a, dW_u = du^T a, da = dg W_g + du W_u
  permutation  dx_t += sum_{k real} da_{p(t,k)}; the shared expert adds its own da.

Only null experts that output zero are covered (copy and constant slots are not).
Pinned in tests/test_oracle_backward.py by central finite differences of L on tiny
float64 layers, with no term retyped from here.
"""
import numpy as np

from oracle import moe_oracle as O

f64 = np.float64


def _swiglu_backward(a, w_gate, w_up, w_down, dY):
    """Gradients of sum <dY, W_down (silu(W_gate a) * W_up a)> for one expert."""
    a = np.asarray(a, f64)
    wg, wu, wd = O._vals(w_gate), O._vals(w_up), O._vals(w_down)
    g = a @ wg.T
    u = a @ wu.T
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    sg = g * sig
    h = sg * u
    dh = dY @ wd
    dwd = dY.T @ h
    dg = dh * u * (sig * (1.0 + g * (1.0 - sig)))
    du = dh * sg
    return dict(dw_gate=dg.T @ a, dw_up=du.T @ a, dw_down=dwd, da=dg @ wg + du @ wu,
                h=h, dh=dh, dg=dg, du=du)


def layer_backward(wl, dy, alpha=0.0, beta=0.0, logits=None):
    """Gradients of L = <dy, y> + alpha L_bal + beta L_z for the layer of ``wl``.
    ``logits`` (T x (N+1), column N the effective null logit) fixes the routing as
    in ``layer_forward``. Returns dx, dw_router ([N+1, d]; row N is zero when M = 0),
    dw_gate / dw_up / dw_down (stacked per expert), the shared expert's dws_* when
    present, and the intermediate ds (logit gradient), dw (per slot weight gradient),
    dy_perm, dx_perm."""
    cfg = wl.cfg
    if cfg.null_kind != "zero":
        raise NotImplementedError("backward covers null experts that output zero")
    N, M, K = cfg.n_experts, cfg.n_null, cfg.top_k
    fwd = O.layer_forward(wl, logits=logits)
    x = wl.values("x")
    wr = wl.values("w_router")
    T, d = x.shape
    dy = np.asarray(dy, f64)
    topk, w, slot_pos = fwd["topk_idx"], fwd["topk_w"], fwd["slot_pos"]
    yp, offsets, perm = fwd["y_perm"], fwd["offsets"], fwd["perm_token"]
    R = yp.shape[0]

    # combine
    dyp = np.zeros((R, d), f64)
    dw = np.zeros((T, K), f64)
    for k in range(K):
        p = slot_pos[:, k]
        m = p >= 0
        dyp[p[m]] = w[m, k][:, None] * dy[m]
        dw[m, k] = (dy[m] * yp[p[m]]).sum(axis=1)

    # renormalised softmax over the chosen reals
    ds = np.zeros((T, N + 1), f64)
    real = topk < N
    gdg = (w * dw * real).sum(axis=1)
    for k in range(K):
        m = real[:, k]
        ds[np.nonzero(m)[0], topk[m, k]] += w[m, k] * (dw[m, k] - gdg[m])

    # auxiliary losses over the pool
    aux = fwd["aux"]
    p, lse = O.pool_softmax(fwd["logits"], N, M)
    f = aux["f"]
    if T:
        fbar = p @ f
        zt = np.where(np.isfinite(lse), lse, 0.0)   # z-loss term of a null at +inf: 0
        dv = alpha * (N / T) * p * (f[None, :] - fbar[:, None]) + beta * (2.0 / T) * zt[:, None] * p
        ds[:, :N] += dv[:, :N]
        if M:
            ds[:, N] += dv[:, N:].sum(axis=1)

    dx = ds @ wr
    dw_router = ds.T @ x

    # routed experts, segment by segment
    xp = x[perm]
    dxp = np.zeros((R, d), f64)
    dwg = np.zeros(np.shape(wl.w_gate), f64)
    dwu = np.zeros(np.shape(wl.w_up), f64)
    dwd = np.zeros(np.shape(wl.w_down), f64)
    for e in range(N):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            continue
        b = _swiglu_backward(xp[lo:hi], wl.w_gate[e], wl.w_up[e], wl.w_down[e], dyp[lo:hi])
        dwg[e], dwu[e], dwd[e] = b["dw_gate"], b["dw_up"], b["dw_down"]
        dxp[lo:hi] = b["da"]
    for k in range(K):
        p_ = slot_pos[:, k]
        m = p_ >= 0
        dx[m] += dxp[p_[m]]

    out = dict(dx=dx, dw_router=dw_router, dw_gate=dwg, dw_up=dwu, dw_down=dwd, ds=ds, dw=dw,
               dy_perm=dyp, dx_perm=dxp, fwd=fwd)
    if cfg.d_ff_shared:
        b = _swiglu_backward(x, wl.ws_gate, wl.ws_up, wl.ws_down, dy)
        dx += b["da"]
        out.update(dws_gate=b["dw_gate"], dws_up=b["dw_up"], dws_down=b["dw_down"])
    return out


def layer_loss(wl, dy, alpha=0.0, beta=0.0):
    """L = <dy, y> + alpha L_bal + beta L_z, evaluated by the forward oracle."""
    fwd = O.layer_forward(wl)
    a = fwd["aux"]
    return float((np.asarray(dy, f64) * fwd["y"]).sum() + alpha * a["L_bal"] + beta * a["L_z"])


def sampled_backward(wl, dy, alpha, beta, logits, tokens, experts):
    """The same gradients restricted to what some outputs depend on, at any size: the
    dx rows of ``tokens`` (their router term, their slots' expert terms and their
    shared-expert term) and the weight gradients of ``experts`` (their segments'
    rows). Routing, permutation and the pool statistics f, p, lse come from the whole
    batch; the expert chains run only on the rows needed. Returns dict(dx [tokens],
    ds [tokens], dw_gate / dw_up / dw_down {expert: matrix})."""
    cfg = wl.cfg
    if cfg.null_kind != "zero":
        raise NotImplementedError("backward covers null experts that output zero")
    N, M, K = cfg.n_experts, cfg.n_null, cfg.top_k
    logits = np.asarray(logits, f64)
    x = wl.values("x")
    wr = wl.values("w_router")
    T = x.shape[0]
    dy = np.asarray(dy, f64)
    topk, w, _ = O.route(logits, N, M, K)
    counts, offsets, perm, slot_pos = O.permute(topk, N)
    aux = O.aux_stats(logits, topk, N, M, K)
    tokens = np.asarray(tokens)
    out = dict(dw_gate={}, dw_up={}, dw_down={})
    for e in experts:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        rows = perm[lo:hi]
        ks = np.array([int(np.nonzero(slot_pos[t] == p)[0][0]) for t, p in zip(rows, range(lo, hi))],
                      dtype=np.int64).reshape(-1)
        dY = w[rows, ks][:, None] * dy[rows] if hi > lo else np.zeros((0, x.shape[1]))
        b = _swiglu_backward(x[rows], wl.w_gate[e], wl.w_up[e], wl.w_down[e], dY)
        out["dw_gate"][e], out["dw_up"][e], out["dw_down"][e] = b["dw_gate"], b["dw_up"], b["dw_down"]
    ds = np.zeros((len(tokens), N + 1), f64)
    dx = np.zeros((len(tokens), x.shape[1]), f64)
    p, lse = O.pool_softmax(logits[tokens], N, M)
    f = aux["f"]
    fbar = p @ f
    zt = np.where(np.isfinite(lse), lse, 0.0)   # z-loss term of a null at +inf: 0
    dv = alpha * (N / T) * p * (f[None, :] - fbar[:, None]) + beta * (2.0 / T) * zt[:, None] * p
    ds[:, :N] = dv[:, :N]
    if M:
        ds[:, N] = dv[:, N:].sum(axis=1)
    for i, t in enumerate(tokens):
        real = [k for k in range(K) if topk[t, k] < N]
        dg = {}
        for k in real:
            e = topk[t, k]
            a = x[t:t + 1]
            dg[k] = float((dy[t] * O.swiglu_ffn(a, wl.w_gate[e], wl.w_up[e], wl.w_down[e])[0]).sum())
            dx[i] += _swiglu_backward(a, wl.w_gate[e], wl.w_up[e], wl.w_down[e], w[t, k] * dy[t:t + 1])["da"][0]
        gdg = sum(w[t, k] * dg[k] for k in real)
        for k in real:
            ds[i, topk[t, k]] += w[t, k] * (dg[k] - gdg)
        if cfg.d_ff_shared:
            dx[i] += _swiglu_backward(x[t:t + 1], wl.ws_gate, wl.ws_up, wl.ws_down, dy[t:t + 1])["da"][0]
    dx += ds @ wr
    out.update(dx=dx, ds=ds)
    return out
