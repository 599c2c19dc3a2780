"""fp64 CPU oracle for TurboT2VA's joint sCM training target.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (no kernels, helpers, tables or constants); both consume the same seeded
inputs, which are drawn by a module that holds none of the method's arithmetic.

What it computes, following "TurboT2VA：分数正则化一致性蒸馏加速 19B 视频音频联合生成"
(robotworld.top Chinese deep read of arXiv 2608.24674; cited below as [deep
read]) and its English condensed read (robotworld.top/en; [English read]):

* TrigFlow noising with a shared timestep and independent noise per modality
  ([deep read] section 3, the noising equation; [English read] section 2).
* A joint block G(z^v, z^a, t, c) producing x0-predictions for both
  modalities in one shared graph ([deep read] section 3, the G_theta equation).
  The 19B backbone is not available; the block is the synthetic one the
  workloads describe (per-modality input projection, sinusoidal time embedding
  through a linear layer, one multi-head self-attention over
  [video; audio; valid text] tokens, per-modality output projection).
* TrigFlow fields F = (cos t z_t - x0_hat)/sin t ([deep read] section 3.1).
* The joint JVP J = c_t (dF/dt + dF/dz^v F_T^v + dF/dz^a F_T^a),
  c_t = cos t sin t ([deep read] section 3.1, the J_theta equation), computed
  here by forward-mode dual numbers pushed through every step of the block,
  including the time embedding ([deep read] section 4.2 requires the JVP to
  pass through the timestep embedding and the cross-modal transformer).
* The sCM direction g, its per-sample per-modality L2 normalisation, the
  residual r and the w_m-weighted joint loss ([deep read] section 3.1; the
  normalisation is "Eq. 6" in [English read] section 2).

Everything is float64.  Inputs are the exact stored (bf16- or fp32-rounded)
values upcast.  Attention is a plain per-query-chunk softmax with the row
maximum subtracted; since softmax is shift invariant, that shift is treated as
a constant in the dual arithmetic, which is exact.
"""
from __future__ import annotations

import math

import numpy as np


# ---------------------------------------------------------------------------
# Optional storage rounding.  With STORAGE = "bf16" the values the GPU path
# stores in bfloat16 between its kernels (noised latents and their tangents,
# the block's token rows, Q/K/V and their tangents, the attention outputs) are
# rounded to bfloat16 here too, so that decisions a near-one-hot softmax takes
# on those values are taken in the same precision on both sides.  The default
# (None) is the exact fp64 oracle.
# ---------------------------------------------------------------------------
STORAGE = None


def _bf16(x):
    """Round float64 values to the nearest bfloat16 (ties to even) via fp32 bits."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _store(x):
    if STORAGE is None:
        return x
    if isinstance(x, Dual):
        return Dual(_bf16(x.p), _bf16(x.t))
    return _bf16(x)


# ---------------------------------------------------------------------------
# Dual numbers: value p and tangent t, pushed forward by the chain rule.
# ---------------------------------------------------------------------------
class Dual:
    __slots__ = ("p", "t")

    def __init__(self, p, t):
        self.p = p
        self.t = t


def const(x) -> Dual:
    x = np.asarray(x, dtype=np.float64)
    return Dual(x, np.zeros_like(x))


def d_add(a: Dual, b: Dual) -> Dual:
    return Dual(a.p + b.p, a.t + b.t)


def d_sub(a: Dual, b: Dual) -> Dual:
    return Dual(a.p - b.p, a.t - b.t)


def d_mul(a: Dual, b: Dual) -> Dual:
    """Product rule: (ab)' = a'b + ab'."""
    return Dual(a.p * b.p, a.t * b.p + a.p * b.t)


def d_scale(a: Dual, s: float) -> Dual:
    return Dual(a.p * s, a.t * s)


def d_div(a: Dual, b: Dual) -> Dual:
    """Quotient rule: (a/b)' = (a'b - ab')/b^2."""
    return Dual(a.p / b.p, (a.t * b.p - a.p * b.t) / (b.p * b.p))


def d_exp(a: Dual) -> Dual:
    e = np.exp(a.p)
    return Dual(e, e * a.t)


def d_cos(a: Dual) -> Dual:
    return Dual(np.cos(a.p), -np.sin(a.p) * a.t)


def d_sin(a: Dual) -> Dual:
    return Dual(np.sin(a.p), np.cos(a.p) * a.t)


def d_matmul(a: Dual, b: Dual) -> Dual:
    """Matrix product, bilinear: (AB)' = A'B + AB'."""
    return Dual(a.p @ b.p, a.t @ b.p + a.p @ b.t)


def d_linear(x: Dual, w: np.ndarray) -> Dual:
    """y = x W^T with a constant weight [out, in] (nn.Linear convention)."""
    return Dual(x.p @ w.T, x.t @ w.T)


def d_T(a: Dual) -> Dual:
    return Dual(a.p.T, a.t.T)


def d_sum(a: Dual, axis, keepdims=False) -> Dual:
    return Dual(a.p.sum(axis=axis, keepdims=keepdims), a.t.sum(axis=axis, keepdims=keepdims))


def d_concat(parts, axis=0) -> Dual:
    return Dual(np.concatenate([x.p for x in parts], axis=axis),
                np.concatenate([x.t for x in parts], axis=axis))


def d_rows(a: Dual, idx) -> Dual:
    return Dual(a.p[idx], a.t[idx])


# ---------------------------------------------------------------------------
# The method's elementwise steps.
# ---------------------------------------------------------------------------
def trigflow_noise(t, z0, eps):
    """z_t = cos(t) z0 + sin(t) eps  ([deep read] section 3, noising equation)."""
    return math.cos(t) * np.asarray(z0, np.float64) + math.sin(t) * np.asarray(eps, np.float64)


def trigflow_field(t, z_t, x0_hat):
    """F = (cos(t) z_t - x0_hat) / sin(t)  ([deep read] section 3.1, field equation).

    ``t``, ``z_t`` and ``x0_hat`` may be Duals (student) or plain arrays (teacher).
    """
    if isinstance(t, Dual):
        return d_div(d_sub(d_mul(d_cos(t), z_t), x0_hat), d_sin(t))
    return (math.cos(t) * np.asarray(z_t, np.float64) - np.asarray(x0_hat, np.float64)) / math.sin(t)


def boost_factor(t, beta, gamma):
    """beta cos(t) / sqrt(1 - gamma^2 sin^2(t)), the weight of the consistency term
    in the sCM direction ([deep read] section 3.1, g_sCM equation)."""
    return beta * math.cos(t) / math.sqrt(1.0 - gamma * gamma * math.sin(t) ** 2)


def scm_direction(t, beta, gamma, F_student, F_teacher, z_t, J):
    """g = -beta cos t / sqrt(1 - gamma^2 sin^2 t) (sg(F_theta) - F_T) - gamma cos t sin t z_t - J.

    sg() is the identity in value ([deep read] section 3.1, g_sCM equation).
    """
    return (-boost_factor(t, beta, gamma) * (F_student - F_teacher)
            - gamma * math.cos(t) * math.sin(t) * z_t - J)


def l2_normalise(g, eps_scm):
    """g / (||g||_2 + eps), the norm taken over every latent element of one sample's
    modality ([deep read] section 3.1; "Eq. 6" of [English read] section 2)."""
    n = math.sqrt(float(np.sum(np.square(g))))
    return g / (n + eps_scm), n


# ---------------------------------------------------------------------------
# The synthetic joint block G and its forward-mode derivative.
# ---------------------------------------------------------------------------
def time_embedding(t: Dual, d: int) -> Dual:
    """Sinusoidal embedding e(t) in R^d: [cos(t w_k) | sin(t w_k)], w_k = 10000^(-k/(d/2))."""
    half = d // 2
    omega = 10000.0 ** (-np.arange(half, dtype=np.float64) / half)
    arg = Dual(t.p * omega, t.t * omega)
    return d_concat([d_cos(arg), d_sin(arg)])


def attention(q: Dual, k: Dual, v: Dual, chunk: int = 512) -> Dual:
    """softmax(q k^T / sqrt(dh)) v for one head, with duals, chunked over queries.

    q [Nq, dh], k/v [Nk, dh]; every key given here is valid (padded keys have
    already been dropped).
    """
    dh = q.p.shape[1]
    scale = 1.0 / math.sqrt(dh)
    kT = d_T(k)
    outs = []
    for s0 in range(0, q.p.shape[0], chunk):
        qc = d_rows(q, slice(s0, s0 + chunk))
        s = d_scale(d_matmul(qc, kT), scale)
        shift = s.p.max(axis=1, keepdims=True)          # constant: softmax is shift invariant
        e = d_exp(Dual(s.p - shift, s.t))
        denom = d_sum(e, axis=1, keepdims=True)
        p = d_div(e, denom)
        outs.append(d_matmul(p, v))
    return d_concat(outs)


def attention_lse(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """log-sum-exp of the scaled logits per query row (natural log)."""
    s = (q @ k.T) / math.sqrt(q.shape[1])
    m = s.max(axis=1)
    return m + np.log(np.exp(s - m[:, None]).sum(axis=1))


def joint_block(zv: Dual, za: Dual, t: Dual, text: np.ndarray, mask: np.ndarray, W: dict,
                H: int, query_rows=None):
    """(x0_hat^v, x0_hat^a) = G(z^v, z^a, t, c)  ([deep read] section 3, G_theta equation).

    ``text`` [Nt, d] enters unprojected with zero tangent (c depends on neither
    t nor z); padded text positions (mask == 0) are dropped from the keys.  Only
    video and audio rows are queried, since only their outputs are consumed.
    ``query_rows`` = (rows_v, rows_a) restricts the queried rows (all keys are
    still used).
    """
    d = W["w_t"].shape[0]
    dh = d // H
    Nv = zv.p.shape[0]
    tau = d_linear(time_embedding(t, d), W["w_t"])
    hv = d_add(d_linear(zv, W["w_in_v"]), Dual(tau.p[None, :], tau.t[None, :]))
    ha = d_add(d_linear(za, W["w_in_a"]), Dual(tau.p[None, :], tau.t[None, :]))
    hv, ha = _store(hv), _store(ha)
    hc = const(text[mask.astype(bool)])
    X = d_concat([hv, ha, hc])
    if query_rows is None:
        Xq = d_concat([hv, ha])
        nqv = Nv
    else:
        rv, ra = query_rows
        Xq = d_concat([d_rows(hv, rv), d_rows(ha, ra)])
        nqv = len(rv)
    w_q, w_k, w_v = W["w_qkv"][:d], W["w_qkv"][d:2 * d], W["w_qkv"][2 * d:]
    Q = _store(d_linear(Xq, w_q))
    K = _store(d_linear(X, w_k))
    V = _store(d_linear(X, w_v))
    heads = []
    for h in range(H):
        sl = slice(h * dh, (h + 1) * dh)
        heads.append(attention(Dual(Q.p[:, sl], Q.t[:, sl]), Dual(K.p[:, sl], K.t[:, sl]),
                               Dual(V.p[:, sl], V.t[:, sl])))
    Y = _store(d_concat(heads, axis=1))
    Gv = d_linear(d_rows(Y, slice(0, nqv)), W["w_out_v"])
    Ga = d_linear(d_rows(Y, slice(nqv, None)), W["w_out_a"])
    return Gv, Ga


# ---------------------------------------------------------------------------
# The block's parameterisation: a direct x0-prediction, or a rectified-flow
# velocity model behind the TrigFlow wrapper.
# ---------------------------------------------------------------------------
def rf_wrap(z: Dual, t: Dual):
    """The TrigFlow -> rectified-flow input map ([deep read] section 4.2):
    z_rf = z / (cos t + sin t), t_rf = sin t / (cos t + sin t), as duals."""
    cs = d_add(d_cos(t), d_sin(t))
    return d_div(z, cs), d_div(d_sin(t), cs)


def rf_x0(z_rf: Dual, t_rf: Dual, v: Dual) -> Dual:
    """x0 from a rectified-flow velocity: with z_rf = (1 - t_rf) x0 + t_rf eps and
    v = eps - x0, x0 = z_rf - t_rf v.  The pages give only the input map; this
    output map is the rectified-flow parameterisation solved for x0."""
    return d_sub(z_rf, d_mul(t_rf, v))


def block_x0(zv: Dual, za: Dual, t: Dual, text, mask, W: dict, H: int, param: str = "x0",
             query_rows=None, block=None):
    """x0-predictions (x0^v, x0^a) of the joint block at TrigFlow inputs (z, t).

    param "x0": the block predicts x0 directly at (z, t).
    param "rf": the block is a rectified-flow velocity model; the TrigFlow
    wrapper feeds it (z_rf, t_rf) and converts its velocity back to x0, so the
    JVP passes through the wrapper, the time embedding and the block
    ([deep read] section 4.2).
    The block's token inputs are what is stored (bf16 in storage mode).
    ``block`` replaces the joint block (same signature) for checks with a stub.
    """
    block = joint_block if block is None else block
    if param == "x0":
        return block(_store(zv), _store(za), t, text, mask, W, H, query_rows=query_rows)
    if param != "rf":
        raise ValueError(param)
    zv_rf, t_rf = rf_wrap(zv, t)
    za_rf, _ = rf_wrap(za, t)
    vv, va = block(_store(zv_rf), _store(za_rf), t_rf, text, mask, W, H, query_rows=query_rows)
    if query_rows is not None:
        zv_rf, za_rf = d_rows(zv_rf, query_rows[0]), d_rows(za_rf, query_rows[1])
    return rf_x0(zv_rf, t_rf, vv), rf_x0(za_rf, t_rf, va)


# ---------------------------------------------------------------------------
# The full target.
# ---------------------------------------------------------------------------
def scm_sample(cfg, data: dict, teacher: dict, student: dict, b: int, beta=None, gamma=None,
               query_rows=None) -> dict:
    """The joint sCM target for sample ``b``.

    Returns the intermediate fields, J, g and (for full rows) the normalised
    direction, residual, norms and per-sample loss.
    """
    beta = cfg.beta if beta is None else beta
    gamma = cfg.gamma if gamma is None else gamma
    t = float(data["t"][b])
    ct, st = math.cos(t), math.sin(t)
    text, mask = data["text"][b], data["text_mask"][b]

    z_t = {"v": trigflow_noise(t, data["z0_v"][b], data["eps_v"][b]),
           "a": trigflow_noise(t, data["z0_a"][b], data["eps_a"][b])}

    param = getattr(cfg, "param", "x0")
    # Teacher: primal forward only.
    gT_v, gT_a = block_x0(const(z_t["v"]), const(z_t["a"]), const(t), text, mask, teacher, cfg.H, param)
    x0_T = {"v": gT_v.p, "a": gT_a.p}
    F_T = {m: trigflow_field(t, z_t[m], x0_T[m]) for m in "va"}

    # Student: dual forward along (dt = 1, dz^v = F_T^v, dz^a = F_T^a, dc = 0).
    td = Dual(np.float64(t), np.float64(1.0))
    zd = {m: Dual(z_t[m], F_T[m]) for m in "va"}
    gS_v, gS_a = block_x0(zd["v"], zd["a"], td, text, mask, student, cfg.H, param, query_rows=query_rows)
    G_S = {"v": gS_v, "a": gS_a}

    if query_rows is not None:
        rv, ra = query_rows
        sel = {"v": rv, "a": ra}
        zd = {m: Dual(zd[m].p[sel[m]], zd[m].t[sel[m]]) for m in "va"}
        F_T_sel = {m: F_T[m][sel[m]] for m in "va"}
        z_sel = {m: z_t[m][sel[m]] for m in "va"}
    else:
        F_T_sel, z_sel = F_T, z_t

    out = dict(t=t, z_t=z_t, x0_T=x0_T, F_T=F_T)
    ct_st = ct * st
    for m in "va":
        F_S = trigflow_field(td, zd[m], G_S[m])              # dual field of the student
        J = ct_st * F_S.t                                     # c_t * dF/ds along the tangent
        g = scm_direction(t, beta, gamma, F_S.p, F_T_sel[m], z_sel[m], J)
        out[f"x0_S_{m}"] = G_S[m].p
        out[f"Gdot_{m}"] = G_S[m].t
        out[f"F_S_{m}"] = F_S.p
        out[f"J_{m}"] = J
        out[f"g_{m}"] = g
    if query_rows is None:
        loss = 0.0
        norms = []
        for m, w in (("v", cfg.w_v), ("a", cfg.w_a)):
            gbar, n = l2_normalise(out[f"g_{m}"], cfg.eps_scm)
            r = (out[f"F_S_{m}"] - out[f"F_S_{m}"]) - gbar   # F - sg(F) - gbar, in value
            out[f"gbar_{m}"] = gbar
            out[f"r_{m}"] = r
            norms.append(n)
            loss += w * float(np.sum(np.square(r)))
        out["norms"] = np.array(norms)
        out["loss"] = loss
    return out


def scm_target(problem: dict, beta=None, gamma=None) -> dict:
    """The joint sCM target for a whole batch; arrays stacked over the batch."""
    cfg, data = problem["cfg"], problem["data"]
    per = [scm_sample(cfg, data, problem["teacher"], problem["student"], b, beta, gamma)
           for b in range(cfg.B)]
    res = {}
    for key in ("J_v", "J_a", "g_v", "g_a", "gbar_v", "gbar_a", "r_v", "r_a", "x0_S_v", "x0_S_a",
                "Gdot_v", "Gdot_a", "F_S_v", "F_S_a"):
        res[key] = np.stack([p[key] for p in per])
    for key in ("z_t", "x0_T", "F_T"):
        for m in "va":
            res[f"{key}_{m}"] = np.stack([p[key][m] for p in per])
    res["norms"] = np.stack([p["norms"] for p in per])
    res["loss"] = np.array([p["loss"] for p in per])
    res["t"] = np.array([p["t"] for p in per])
    return res


def student_field(cfg, data, student, b, zv, za, t):
    """Primal student field F_theta(z^v, z^a, t) at an arbitrary point (for derivative checks)."""
    text, mask = data["text"][b], data["text_mask"][b]
    gv, ga = block_x0(const(zv), const(za), const(t), text, mask, student, cfg.H,
                      getattr(cfg, "param", "x0"))
    return trigflow_field(t, zv, gv.p), trigflow_field(t, za, ga.p)


# ---------------------------------------------------------------------------
# Attention forward + JVP on raw operands (layout [B, N, H, dh]).
# ---------------------------------------------------------------------------
def attention_fwd_jvp(q, k, v, qd, kd, vd, nk, query_rows=None):
    """Per (sample, head): O = softmax(Q K^T / sqrt(dh)) V over the first nk[b]
    keys and its tangent dO along (dQ, dK, dV); also the natural-log
    log-sum-exp of the scaled logits.  Returns arrays [B, Nq, H, dh] and [B, H, Nq].
    """
    B, Nq, H, dh = q.shape
    rows = np.arange(Nq) if query_rows is None else np.asarray(query_rows)
    o = np.zeros((B, len(rows), H, dh))
    od = np.zeros_like(o)
    lse = np.zeros((B, H, len(rows)))
    for b in range(B):
        n = int(nk[b])
        for h in range(H):
            Q = Dual(q[b, rows, h].astype(np.float64), qd[b, rows, h].astype(np.float64))
            K = Dual(k[b, :n, h].astype(np.float64), kd[b, :n, h].astype(np.float64))
            V = Dual(v[b, :n, h].astype(np.float64), vd[b, :n, h].astype(np.float64))
            res = attention(Q, K, V)
            o[b, :, h], od[b, :, h] = res.p, res.t
            lse[b, h] = attention_lse(Q.p, K.p)
    return o, od, lse
