"""Pins for the fp64 oracle, independent of the oracle's own code.

The oracle (oracle/gdr_oracle.c) is a token-by-token recurrence plus a
hand-derived reverse. Here it is checked against things that do not reuse its
formulas:
  * central finite differences of its own forward objective (pins the reverse
    recurrence term by term: a dropped term, sign or transposed operand in the
    reverse shows up as an FD mismatch);
  * an independent chunked forward in the WY form that the FlashQLA issue #30
    page's fused_bwd.py decomposes (U = K S, W = V - U, V' = A W with a
    gate-decay mask, state update with the chunk-end decay) and that the
    kernel_fun bwd_intra page's Aqk/Akk inputs presuppose; it also asserts the
    exponent law (every exp2 argument <= 0);
  * closed forms at beta = 0 (the state only decays: S_t = Diag(2^{G_t}) h0);
    with g = 0 as well this is plain (unnormalised, causal) linear attention;
  * decompositions: per-channel gate with equal channels == scalar gate, GQA ==
    duplicated heads summed, packed varlen == separate sequences, linearity of
    every gradient in (do, dht).
"""
import math

import numpy as np
import pytest

LN2 = math.log(2.0)


def rand_case(seed, B=1, T=7, H=2, Hg=1, K=4, V=3, gate="kda", gmult=0.5,
              h0=True, dht=True, cu=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, Hg, K))
    k = rng.standard_normal((B, T, Hg, K))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, V))
    gshape = (B, T, H, K) if gate == "kda" else (B, T, H)
    g = -np.log1p(np.exp(rng.standard_normal(gshape))) * gmult
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    N = B if cu is None else len(cu) - 1
    d = dict(q=q, k=k, v=v, g=g, beta=beta,
             do=rng.standard_normal((B, T, H, V)),
             h0=rng.standard_normal((N, H, K, V)) * 0.5 if h0 else None,
             dht=rng.standard_normal((N, H, K, V)) * 0.5 if dht else None,
             cu_seqlens=None if cu is None else np.asarray(cu, dtype=np.int32),
             scale=K ** -0.5, gate=gate)
    return d


def call(oracle, d, **kw):
    args = dict(d)
    args.update(kw)
    return oracle.run(args["q"], args["k"], args["v"], args["g"], args["beta"],
                      args.get("do"), args.get("h0"), args.get("dht"),
                      args.get("cu_seqlens"), args.get("scale"), args["gate"],
                      backward=kw.get("backward", True),
                      forward_out=kw.get("forward_out", False),
                      chunk=kw.get("chunk", 0))


def loss(oracle, d):
    return oracle.loss(d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"], d["h0"],
                       d["dht"], d["cu_seqlens"], d["scale"], d["gate"])


FD_CASES = [
    dict(seed=1, T=1, gate="kda"),
    dict(seed=2, T=7, gate="kda"),
    dict(seed=3, T=13, gate="gdn", K=3, V=5),
    dict(seed=4, T=13, gate="kda", H=2, Hg=2, K=5, V=4, h0=False),
    dict(seed=5, T=11, gate="kda", cu=[0, 4, 5, 11]),          # varlen, a length-1 sequence
    dict(seed=6, T=9, gate="gdn", cu=[0, 1, 9], dht=False),
    dict(seed=7, B=2, T=5, gate="kda", H=4, Hg=2, K=3, V=3),
]


@pytest.mark.parametrize("case", FD_CASES, ids=lambda c: f"seed{c['seed']}")
def test_reverse_matches_central_fd(oracle_mod, case):
    d = rand_case(**case)
    grads = call(oracle_mod, d)
    eps = 1e-6
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "db", "h0": "dh0"}
    for x, gname in names.items():
        if d[x] is None:
            continue
        fd = np.zeros_like(d[x])
        it = np.nditer(d[x], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            orig = d[x][idx]
            d[x][idx] = orig + eps
            lp = loss(oracle_mod, d)
            d[x][idx] = orig - eps
            lm = loss(oracle_mod, d)
            d[x][idx] = orig
            fd[idx] = (lp - lm) / (2 * eps)
        ref = max(np.abs(fd).max(), 1e-3)
        err = np.abs(fd - grads[gname]).max() / ref
        assert err < 1e-7, f"{gname}: max rel err {err:.3e}"


def test_fd_long_sequence_sampled(oracle_mod):
    """T = 70 spans many decays; sample coordinates rather than all."""
    d = rand_case(seed=11, T=70, K=5, V=4, gate="kda")
    grads = call(oracle_mod, d)
    rng = np.random.default_rng(0)
    eps = 1e-6
    for x, gname in {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "db",
                     "h0": "dh0"}.items():
        flat = d[x].reshape(-1)
        for i in rng.choice(flat.size, size=12, replace=False):
            orig = flat[i]
            flat[i] = orig + eps
            lp = loss(oracle_mod, d)
            flat[i] = orig - eps
            lm = loss(oracle_mod, d)
            flat[i] = orig
            fd = (lp - lm) / (2 * eps)
            scale = max(np.abs(grads[gname]).max(), 1e-3)
            assert abs(fd - grads[gname].reshape(-1)[i]) / scale < 1e-7, gname


# ----------------------------------------------------------------------------
# independent chunked WY forward
# ----------------------------------------------------------------------------

def chunked_forward(d, C):
    """fp64 chunkwise forward in the WY form, per (sequence, head), written
    from the chunk equations (not from the token recurrence):
      G = in-chunk inclusive cumsum of g; Gam = 2^G
      Akk[r,s] = beta_r sum_d k_rd k_sd 2^(G_rd - G_sd)   (s < r)
      Aqk[r,s] = sum_d q_rd k_sd 2^(G_rd - G_sd)           (s <= r)
      A = (I + Akk)^-1 ; w = A (beta k Gam) ; u = A (beta v) ; X = u - w S
      o = scale [ (q Gam) S + Aqk X ]
      S <- Diag(2^G_last) S + (k 2^(G_last - G))^T X
    Every exponent that reaches exp2 is asserted <= 0.
    """
    q, k, v, g, beta = d["q"], d["k"], d["v"], d["g"], d["beta"]
    B, T, Hg, K = q.shape
    H, V = v.shape[2], v.shape[3]
    cu = d["cu_seqlens"]
    seqs = [(b, 0, T) for b in range(B)] if cu is None else \
        [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    o = np.zeros((B, T, H, V))
    ht = np.zeros((len(seqs), H, K, V))
    max_arg = -np.inf
    for n, (b, t0, t1) in enumerate(seqs):
        for h in range(H):
            hk = h // (H // Hg)
            S = d["h0"][n, h].copy() if d["h0"] is not None else np.zeros((K, V))
            for c0 in range(t0, t1, C):
                c1 = min(c0 + C, t1)
                L = c1 - c0
                qc, kc = q[b, c0:c1, hk], k[b, c0:c1, hk]
                vc, bc = v[b, c0:c1, h], beta[b, c0:c1, h]
                gc = g[b, c0:c1, h]
                if gc.ndim == 1:
                    gc = np.repeat(gc[:, None], K, axis=1)
                G = np.cumsum(gc, axis=0)
                Akk = np.zeros((L, L))
                Aqk = np.zeros((L, L))
                for r in range(L):
                    for s in range(r + 1):
                        arg = G[r] - G[s]
                        max_arg = max(max_arg, arg.max())
                        e = np.exp2(arg)
                        Aqk[r, s] = np.sum(qc[r] * kc[s] * e)
                        if s < r:
                            Akk[r, s] = bc[r] * np.sum(kc[r] * kc[s] * e)
                A = np.linalg.solve(np.eye(L) + Akk, np.eye(L))
                max_arg = max(max_arg, G.max())
                Gam = np.exp2(G)
                w = A @ (bc[:, None] * kc * Gam)
                u = A @ (bc[:, None] * vc)
                X = u - w @ S
                o[b, c0:c1, h] = d["scale"] * ((qc * Gam) @ S + Aqk @ X)
                arg = G[-1][None, :] - G
                max_arg = max(max_arg, arg.max())
                S = np.exp2(G[-1])[:, None] * S + (kc * np.exp2(arg)).T @ X
            ht[n, h] = S
    return o, ht, max_arg


@pytest.mark.parametrize("C", [4, 16, 64])
@pytest.mark.parametrize("gate", ["kda", "gdn"])
def test_forward_matches_chunked_wy(oracle_mod, C, gate):
    for case in (dict(seed=21, B=2, T=77, H=2, Hg=1, K=6, V=5),
                 dict(seed=22, T=70, H=2, Hg=2, K=4, V=4, cu=[0, 1, 18, 19, 70])):
        d = rand_case(gate=gate, **case)
        f = call(oracle_mod, d, backward=False, forward_out=True)
        o, ht, max_arg = chunked_forward(d, C)
        assert max_arg <= 0.0, "exponent law violated"
        assert np.abs(f["o"] - o).max() <= 1e-12 * max(1.0, np.abs(o).max())
        assert np.abs(f["ht"] - ht).max() <= 1e-12 * max(1.0, np.abs(ht).max())


def test_large_gates_exponent_law(oracle_mod):
    """Gates x16: the chunked form still agrees and never exponentiates a
    positive number (the decays underflow instead of overflowing)."""
    d = rand_case(seed=23, T=64, K=4, V=4, gate="kda", gmult=8.0)
    f = call(oracle_mod, d, backward=False, forward_out=True)
    o, ht, max_arg = chunked_forward(d, 16)
    assert max_arg <= 0.0
    assert np.all(np.isfinite(f["o"]))
    assert np.abs(f["o"] - o).max() <= 1e-12 * max(1.0, np.abs(o).max())


# ----------------------------------------------------------------------------
# closed forms at beta = 0
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("gate", ["kda", "gdn"])
@pytest.mark.parametrize("zero_gate", [False, True])
def test_beta_zero_closed_forms(oracle_mod, gate, zero_gate):
    d = rand_case(seed=31, T=9, H=1, Hg=1, K=4, V=3, gate=gate)
    d["beta"][:] = 0.0
    if zero_gate:
        d["g"][:] = 0.0
    q, k, v, do = d["q"][0, :, 0], d["k"][0, :, 0], d["v"][0, :, 0], d["do"][0, :, 0]
    h0, dht, sc = d["h0"][0, 0], d["dht"][0, 0], d["scale"]
    g = d["g"][0, :, 0]
    if g.ndim == 1:
        g = np.repeat(g[:, None], 4, axis=1)
    T = q.shape[0]
    G = np.cumsum(g, axis=0)                      # from the sequence start
    Gam = np.exp2(G)
    out = call(oracle_mod, d, forward_out=True)
    # forward: S_t = Diag(Gam_t) h0
    o_ref = sc * (q * Gam) @ h0
    assert np.allclose(out["o"][0, :, 0], o_ref, rtol=0, atol=1e-13)
    assert np.allclose(out["ht"][0, 0], Gam[-1][:, None] * h0, atol=1e-13)
    # gradients
    assert np.abs(out["dk"]).max() == 0.0 and np.abs(out["dv"]).max() == 0.0
    dq_ref = sc * Gam * (do @ h0.T)
    assert np.allclose(out["dq"][0, :, 0], dq_ref, atol=1e-13)
    dh0_ref = sc * ((q * Gam).T @ do) + Gam[-1][:, None] * dht
    assert np.allclose(out["dh0"][0, 0], dh0_ref, atol=1e-12)
    # db_t = k_t^T Lam_t e_t with Lam_t = dL/dS_t, e_t = v_t - h0^T Diag(Gam_t) k_t
    db_ref = np.zeros(T)
    dg_ref = np.zeros((T, 4))
    for t in range(T):
        lam = sc * sum(np.exp2(G[u] - G[t])[:, None] * np.outer(q[u], do[u])
                       for u in range(t, T)) + np.exp2(G[-1] - G[t])[:, None] * dht
        e = v[t] - h0.T @ (Gam[t] * k[t])
        db_ref[t] = k[t] @ lam @ e
        # dL/dg_t[d] = ln2 * sum over every term whose exponent contains g_t
        dg_ref[t] = LN2 * (sum(sc * q[u] * Gam[u] * (h0 @ do[u]) for u in range(t, T))
                           + Gam[-1] * np.sum(dht * h0, axis=1))
    assert np.allclose(out["db"][0, :, 0], db_ref, atol=1e-12)
    dg = out["dg"][0, :, 0]
    if gate == "gdn":
        dg_ref = dg_ref.sum(axis=1)
    assert np.allclose(dg, dg_ref, atol=1e-12)
    if zero_gate:
        # plain causal linear attention: db_t = scale sum_{u>=t} (q_u.k_t)(do_u.vt_t)
        #                                       + k_t^T dht vt_t,  vt_t = v_t - h0^T k_t
        vt = v - k @ h0
        la = sc * np.tril(q @ k.T) * (do @ vt.T)      # [u, t] for u >= t
        db_la = la.sum(axis=0) + np.einsum("tk,kv,tv->t", k, dht, vt)
        assert np.allclose(out["db"][0, :, 0], db_la, atol=1e-12)


def test_single_token_by_hand(oracle_mod):
    """T = 1, K = V = 1: every gradient written out by hand."""
    q, k, v, g, b, h0, do, dht, sc = 0.7, -1.3, 0.4, -0.6, 0.3, 0.9, 1.1, -0.5, 0.8
    a = 2.0 ** g
    P = a * h0
    e = v - P * k
    S = P + b * k * e
    lam = dht + sc * q * do
    de = b * lam * k
    ref = dict(dq=sc * S * do, db=k * lam * e, dv=de, dk=b * lam * e - P * de,
               dg=LN2 * a * (lam - k * de) * h0, dh0=a * (lam - k * de))
    arr = lambda x, *s: np.full(s, x, dtype=np.float64)
    out = oracle_mod.run(arr(q, 1, 1, 1, 1), arr(k, 1, 1, 1, 1), arr(v, 1, 1, 1, 1),
                         arr(g, 1, 1, 1, 1), arr(b, 1, 1, 1), arr(do, 1, 1, 1, 1),
                         arr(h0, 1, 1, 1, 1), arr(dht, 1, 1, 1, 1), None, sc, "kda",
                         forward_out=True)
    assert abs(out["o"].item() - sc * S * q) < 1e-15
    for name, val in ref.items():
        assert abs(out[name].item() - val) < 1e-14, name


# ----------------------------------------------------------------------------
# decompositions
# ----------------------------------------------------------------------------

def test_channel_constant_kda_equals_gdn(oracle_mod):
    d = rand_case(seed=41, T=20, H=2, Hg=1, K=4, V=3, gate="gdn")
    ref = call(oracle_mod, d)
    dk = dict(d)
    dk["gate"] = "kda"
    dk["g"] = np.repeat(d["g"][..., None], 4, axis=-1)
    out = call(oracle_mod, dk)
    for n in ("dq", "dk", "dv", "db", "dh0"):
        assert np.allclose(out[n], ref[n], atol=1e-13), n
    assert np.allclose(out["dg"].sum(-1), ref["dg"], atol=1e-13)


def test_gqa_equals_duplicated_heads(oracle_mod):
    d = rand_case(seed=42, T=15, H=4, Hg=2, K=3, V=4, gate="kda")
    ref = call(oracle_mod, d)
    dd = dict(d)
    dd["q"] = np.repeat(d["q"], 2, axis=2)
    dd["k"] = np.repeat(d["k"], 2, axis=2)
    out = call(oracle_mod, dd)
    for n in ("dv", "dg", "db", "dh0"):
        assert np.allclose(out[n], ref[n], atol=1e-13), n
    for n in ("dq", "dk"):
        summed = out[n].reshape(1, 15, 2, 2, 3).sum(axis=3)
        assert np.allclose(summed, ref[n], atol=1e-13), n


def test_varlen_equals_separate_sequences(oracle_mod):
    cu = [0, 5, 6, 19, 30]
    d = rand_case(seed=43, T=30, H=2, Hg=1, K=3, V=3, gate="kda", cu=cu)
    ref = call(oracle_mod, d)
    for n in range(len(cu) - 1):
        t0, t1 = cu[n], cu[n + 1]
        s = dict(d)
        for x in ("q", "k", "v", "g", "beta", "do"):
            s[x] = d[x][:, t0:t1]
        s["h0"] = d["h0"][n:n + 1]
        s["dht"] = d["dht"][n:n + 1]
        s["cu_seqlens"] = None
        out = call(oracle_mod, s)
        for name in ("dq", "dk", "dv", "dg", "db"):
            assert np.allclose(out[name], ref[name][:, t0:t1], atol=1e-13), name
        assert np.allclose(out["dh0"][0], ref["dh0"][n], atol=1e-13)


def test_linear_in_output_gradients(oracle_mod):
    d1 = rand_case(seed=44, T=12, gate="kda")
    d2 = rand_case(seed=45, T=12, gate="kda")
    a, b = 0.7, -1.9
    d3 = dict(d1)
    d3["do"] = a * d1["do"] + b * d2["do"]
    d3["dht"] = a * d1["dht"] + b * d2["dht"]
    d2 = dict(d1, do=d2["do"], dht=d2["dht"])
    r1, r2, r3 = call(oracle_mod, d1), call(oracle_mod, d2), call(oracle_mod, d3)
    for n in ("dq", "dk", "dv", "dg", "db", "dh0"):
        assert np.allclose(r3[n], a * r1[n] + b * r2[n], atol=1e-12), n


def test_chunk_boundary_states(oracle_mod):
    """The per-chunk states the oracle exposes agree with shorter runs: the state
    before chunk c equals ht of the prefix, and dL/dS at the end of chunk c
    equals dh0 of the suffix problem that starts there."""
    C = 8
    d = rand_case(seed=46, T=27, H=1, Hg=1, K=3, V=3, gate="kda")
    out = call(oracle_mod, d, chunk=C)
    f = call(oracle_mod, d, backward=False, forward_out=True)
    for c in range(4):
        t0 = c * C
        pre = dict(d)
        for x in ("q", "k", "v", "g", "beta", "do"):
            pre[x] = d[x][:, :t0] if t0 > 0 else d[x][:, :0]
        if t0 == 0:
            assert np.allclose(out["h_chunks"][0, 0], d["h0"][0, 0])
            continue
        fp = call(oracle_mod, pre, backward=False, forward_out=True)
        assert np.allclose(out["h_chunks"][c, 0], fp["ht"][0, 0], atol=1e-13)
    for c in range(4):
        t1 = min((c + 1) * C, 27)
        suf = dict(d)
        for x in ("q", "k", "v", "g", "beta", "do"):
            suf[x] = d[x][:, t1:]
        if t1 == 27:
            assert np.allclose(out["dh_chunks"][c, 0], d["dht"][0, 0])
            continue
        # the suffix problem starts from the true state S_{t1}
        fpre = dict(d)
        for x in ("q", "k", "v", "g", "beta", "do"):
            fpre[x] = d[x][:, :t1]
        st = call(oracle_mod, fpre, backward=False, forward_out=True)["ht"]
        suf["h0"] = st
        rs = call(oracle_mod, suf)
        assert np.allclose(out["dh_chunks"][c, 0], rs["dh0"][0, 0], atol=1e-12)
    assert np.allclose(f["ht"], call(oracle_mod, d, backward=False, forward_out=True)["ht"])
