"""Pins that tie the CPU oracle to what the pages and the mathematics fix.

Each pin takes the oracle module ``o`` so that the mutation tests can hand in a
copy with a planted mistake and check that some pin catches it.  No pin
re-types the oracle's formula: each one uses a closed form, an invariant, a
brute-force loop over tiny inputs, or an independent library routine (PyTorch
CPU) for a special case.
"""
from __future__ import annotations

import math
from types import SimpleNamespace

import numpy as np
import torch

F64 = np.float64


def _rng(seed):
    return np.random.default_rng(seed)


def dims(D=16, Hq=4, Hkv=2, d=8, F=24, eps=1e-6):
    return SimpleNamespace(D=D, Hq=Hq, Hkv=Hkv, d=d, F=F, eps=eps)


def rand_layers(rng, dm, L, std=0.3, gain_std=0.2):
    D, Hq, Hkv, d, F = dm.D, dm.Hq, dm.Hkv, dm.d, dm.F
    out = []
    for _ in range(L):
        out.append(dict(
            w_qkv=rng.normal(0, std, ((Hq + 2 * Hkv) * d, D)),
            w_o=rng.normal(0, std, (D, Hq * d)),
            w_gateup=rng.normal(0, std, (2 * F, D)),
            w_down=rng.normal(0, std, (D, F)),
            g_attn=1 + rng.normal(0, gain_std, D),
            g_ffn=1 + rng.normal(0, gain_std, D),
        ))
    return out


def cache_with(o, L, B, Hkv, d, lens, rng):
    c = o.OracleCache(L, B, Hkv, d)
    for l in range(L):
        for b in range(B):
            c.append(l, b, rng.normal(0, 1, (lens[b], Hkv, d)), rng.normal(0, 1, (lens[b], Hkv, d)))
    return c


# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------
def pin_bf16_values(o):
    # Hand-worked values: bf16 keeps 8 significant bits; ties go to the even mantissa.
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8 + 2 ** -20), 3.0, 0.0,
                  2 ** -130 * 3, 65504.0])
    want = np.array([1.0, 1.0, 1 + 2 ** -6, -(1 + 2 ** -7), 3.0, 0.0, 2 ** -130 * 3, 65536.0])
    got = o.to_bf16(x)
    assert np.array_equal(got, want), (got, want)


def pin_bf16_vs_torch(o):
    # Special case reducing to a library routine: fp32 -> bf16 conversion in torch.
    x = _rng(1).normal(0, 3, 4096).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(o.to_bf16(x.astype(F64)), ref)
    assert np.array_equal(o.store(x.astype(F64), "f32"), x.astype(F64))


# ---------------------------------------------------------------------------
# elementwise
# ---------------------------------------------------------------------------
def pin_rmsnorm_torch(o):
    rng = _rng(2)
    x = rng.normal(0, 2, (5, 32))
    g = 1 + rng.normal(0, 0.3, 32)
    m = torch.nn.RMSNorm(32, eps=1e-6, dtype=torch.float64)
    with torch.no_grad():
        m.weight.copy_(torch.from_numpy(g))
        ref = m(torch.from_numpy(x)).numpy()
    assert np.allclose(o.rmsnorm(x, g, 1e-6), ref, rtol=1e-13, atol=1e-13)


def pin_rmsnorm_invariant(o):
    # mean((y/g)^2) = ms / (ms + eps) exactly in real arithmetic.
    rng = _rng(3)
    x = rng.normal(0, 0.01, (7, 64))         # small ms so eps matters
    g = 1 + rng.normal(0, 0.3, 64)
    eps = 1e-4
    y = o.rmsnorm(x, g, eps)
    ms = np.mean(x * x, axis=1)
    assert np.allclose(np.mean((y / g) ** 2, axis=1), ms / (ms + eps), rtol=1e-12)


def pin_silu(o):
    x = np.linspace(-12, 12, 241)
    ref = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    assert np.allclose(o.silu(x), ref, rtol=1e-14, atol=1e-15)
    assert o.silu(np.array([0.0]))[0] == 0.0


# ---------------------------------------------------------------------------
# (a) fusion
# ---------------------------------------------------------------------------
def pin_fuse_selector(o):
    # W_c = [0 .. I .. 0] with the identity in block k: H_t = RMSNorm(H(l_k)).
    rng = _rng(4)
    T, D, n = 6, 16, 5
    hs = [rng.normal(0, 1 + k, (T, D)) for k in range(n)]
    g = 1 + rng.normal(0, 0.2, D)
    for k in range(n):
        w = np.zeros((D, n * D))
        w[:, k * D:(k + 1) * D] = np.eye(D)
        got = o.fuse_context(hs, w, g, 1e-6, "f32")
        ms = np.mean(hs[k] ** 2, axis=1, keepdims=True)
        want = (g * hs[k] / np.sqrt(ms + 1e-6)).astype(np.float32).astype(F64)
        assert np.allclose(got, want, rtol=1e-6, atol=1e-7), k


def pin_fuse_torch_linear(o):
    # Library routine: torch Linear(5D -> D, no bias) then RMSNorm, on tiny shapes.
    rng = _rng(5)
    T, D, n = 9, 16, 5
    hs = [rng.normal(0, 1, (T, D)) for _ in range(n)]
    w = rng.normal(0, 0.1, (D, n * D))
    g = 1 + rng.normal(0, 0.2, D)
    lin = torch.nn.Linear(n * D, D, bias=False, dtype=torch.float64)
    nrm = torch.nn.RMSNorm(D, eps=1e-6, dtype=torch.float64)
    with torch.no_grad():
        lin.weight.copy_(torch.from_numpy(w))
        nrm.weight.copy_(torch.from_numpy(g))
        ref = nrm(lin(torch.cat([torch.from_numpy(h) for h in hs], dim=-1))).numpy()
    got = o.fuse_context(hs, w, g, 1e-6, "bf16")
    # bf16 storage: within half an ulp (2^-9 relative) of the exact value
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-30)
    assert np.array_equal(got, o.to_bf16(got))


# ---------------------------------------------------------------------------
# (b) injection
# ---------------------------------------------------------------------------
def pin_inject_identity(o):
    # D = Hkv*d, W_K = I and W_V = 2I: cache K rows equal H_t, V rows 2*H_t, and
    # the W_Q rows (NaN here) are never used.
    Hkv, d = 2, 8
    D = Hkv * d
    T = 5
    H = np.arange(T * D, dtype=F64).reshape(T, D) / 7.0     # position-coded rows
    want_k = H.astype(np.float32).astype(F64)
    want_v = (2 * H).astype(np.float32).astype(F64)
    for Hq in (Hkv, 2 * Hkv):
        w = np.concatenate([np.full((Hq * d, D), np.nan), np.eye(D), 2 * np.eye(D)], axis=0)
        k, v = o.inject_kv(H, w, Hq, Hkv, d, "f32")
        assert k.shape == (T, Hkv, d) and v.shape == (T, Hkv, d)
        assert np.array_equal(k.reshape(T, D), want_k)
        assert np.array_equal(v.reshape(T, D), want_v)
        # head-major split: head j of row t holds H[t, j*d:(j+1)*d]
        assert np.array_equal(k[3, 1], want_k[3, d:2 * d])


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def _brute_attention(q, k, v):
    # Pure-Python loops, float64.
    R, Hq, d = q.shape
    n, Hkv, _ = k.shape
    G = Hq // Hkv
    out = np.zeros((R, Hq, d))
    for r in range(R):
        for h in range(Hq):
            j = h // G
            s = [sum(q[r, h, c] * k[t, j, c] for c in range(d)) / math.sqrt(d) for t in range(n)]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            z = sum(e)
            for c in range(d):
                out[r, h, c] = sum(e[t] * v[t, j, c] for t in range(n)) / z
    return out


def pin_attention_bruteforce(o):
    rng = _rng(7)
    for (R, Hq, Hkv, d, n) in [(3, 4, 2, 4, 6), (4, 2, 2, 3, 1), (2, 6, 3, 5, 8)]:
        q = rng.normal(0, 1, (R, Hq, d))
        k = rng.normal(0, 1, (n, Hkv, d))
        v = rng.normal(0, 1, (n, Hkv, d))
        assert np.allclose(o.attention(q, k, v), _brute_attention(q, k, v), rtol=1e-12, atol=1e-12)


def pin_attention_closed_forms(o):
    rng = _rng(8)
    R, Hq, Hkv, d, n = 4, 4, 2, 8, 9
    q = rng.normal(0, 1, (R, Hq, d))
    k = rng.normal(0, 1, (n, Hkv, d))
    # equal value rows -> output equals that row
    vrow = rng.normal(0, 1, (Hkv, d))
    v = np.broadcast_to(vrow, (n, Hkv, d)).copy()
    out = o.attention(q, k, v)
    for h in range(Hq):
        assert np.allclose(out[:, h], vrow[h // (Hq // Hkv)], atol=1e-12)
    # Q = 0 -> mean of the value rows
    v = rng.normal(0, 1, (n, Hkv, d))
    out = o.attention(np.zeros_like(q), k, v)
    for h in range(Hq):
        assert np.allclose(out[:, h], v[:, h // (Hq // Hkv)].mean(axis=0), atol=1e-12)
    # single key -> its value row
    out = o.attention(q, k[:1], v[:1])
    for h in range(Hq):
        assert np.allclose(out[:, h], v[0, h // (Hq // Hkv)], atol=1e-12)


def pin_attention_sdpa(o):
    # Library routine: torch SDPA with grouped KV heads (expanded per group).
    rng = _rng(9)
    R, Hq, Hkv, d, n = 5, 8, 2, 16, 11
    q = rng.normal(0, 1, (R, Hq, d))
    k = rng.normal(0, 1, (n, Hkv, d))
    v = rng.normal(0, 1, (n, Hkv, d))
    G = Hq // Hkv
    tq = torch.from_numpy(q).permute(1, 0, 2)                              # [Hq, R, d]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, dim=0)  # [Hq, n, d]
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).permute(1, 0, 2).numpy()
    assert np.allclose(o.attention(q, k, v), ref, rtol=1e-12, atol=1e-12)


def pin_attention_permutations(o):
    rng = _rng(10)
    R, Hq, Hkv, d, n = 6, 4, 1, 8, 12
    q = rng.normal(0, 1, (R, Hq, d))
    k = rng.normal(0, 1, (n, Hkv, d))
    v = rng.normal(0, 1, (n, Hkv, d))
    base = o.attention(q, k, v)
    p = rng.permutation(n)
    assert np.allclose(o.attention(q, k[p], v[p]), base, atol=1e-12)
    pr = rng.permutation(R)
    assert np.allclose(o.attention(q[pr], k, v), base[pr], atol=1e-12)


# ---------------------------------------------------------------------------
# draft forward
# ---------------------------------------------------------------------------
def _torch_layer_forward(dm, layers, g_final, ctx_k, ctx_v, h0):
    """Library-routine composition (float64 CPU): RMSNorm modules, SDPA over the
    joined [context; block] keys with grouped heads, SiLU; one sequence, f32 storage
    of the block K/V is emulated by float32 round trips."""
    D, Hq, Hkv, d, F, eps = dm.D, dm.Hq, dm.Hkv, dm.d, dm.F, dm.eps
    G = Hq // Hkv
    h = torch.from_numpy(h0.copy())
    g_ = h.shape[0]

    def norm(x, g):
        m = torch.nn.RMSNorm(D, eps=eps, dtype=torch.float64)
        with torch.no_grad():
            m.weight.copy_(torch.from_numpy(np.asarray(g, dtype=F64)))
            return m(x)

    with torch.no_grad():
        for l, w in enumerate(layers):
            a = norm(h, w["g_attn"])
            wq = torch.from_numpy(w["w_qkv"][: Hq * d])
            wk = torch.from_numpy(w["w_qkv"][Hq * d:(Hq + Hkv) * d])
            wv = torch.from_numpy(w["w_qkv"][(Hq + Hkv) * d:])
            q = torch.nn.functional.linear(a, wq).reshape(g_, Hq, d).permute(1, 0, 2)
            kb = torch.nn.functional.linear(a, wk).float().double().reshape(g_, Hkv, d)
            vb = torch.nn.functional.linear(a, wv).float().double().reshape(g_, Hkv, d)
            K = torch.cat([torch.from_numpy(ctx_k[l]), kb], 0).permute(1, 0, 2).repeat_interleave(G, 0)
            Vv = torch.cat([torch.from_numpy(ctx_v[l]), vb], 0).permute(1, 0, 2).repeat_interleave(G, 0)
            att = torch.nn.functional.scaled_dot_product_attention(q, K, Vv)      # [Hq, g, d]
            att = att.permute(1, 0, 2).reshape(g_, Hq * d)
            h = h + torch.nn.functional.linear(att, torch.from_numpy(w["w_o"]))
            f = norm(h, w["g_ffn"])
            gu = torch.nn.functional.linear(f, torch.from_numpy(w["w_gateup"]))
            s = torch.nn.functional.silu(gu[:, :F]) * gu[:, F:]
            h = h + torch.nn.functional.linear(s, torch.from_numpy(w["w_down"]))
        return norm(h, g_final).numpy()


def pin_draft_torch_composition(o):
    rng = _rng(11)
    dm = dims()
    L, B, gamma = 2, 2, 5
    layers = rand_layers(rng, dm, L)
    gf = 1 + rng.normal(0, 0.2, dm.D)
    lens = [7, 0]
    cache = cache_with(o, L, B, dm.Hkv, dm.d, lens, rng)
    h0 = rng.normal(0, 1, (B, gamma, dm.D))
    got, _ = o.draft_forward(dm, layers, gf, cache, gamma, override=h0, storage="f32")
    for b in range(B):
        ref = _torch_layer_forward(dm, layers, gf, [cache.k[l][b] for l in range(L)],
                                   [cache.v[l][b] for l in range(L)], h0[b])
        assert np.allclose(got[b], ref, rtol=1e-9, atol=1e-9), b


def pin_draft_zero_branches(o):
    # W_O = 0 and W_down = 0: the residual stream passes through unchanged, so
    # h_final = RMSNorm(embedding; g_final) and logits = E . that, in closed form.
    rng = _rng(12)
    dm = dims()
    L, B, gamma, V = 3, 2, 4, 40
    layers = rand_layers(rng, dm, L)
    for w in layers:
        w["w_o"][:] = 0
        w["w_down"][:] = 0
    gf = 1 + rng.normal(0, 0.2, dm.D)
    E = rng.normal(0, 1, (V, dm.D))
    tok = rng.integers(0, V, (B, gamma))
    cache = cache_with(o, L, B, dm.Hkv, dm.d, [3, 5], rng)
    got, _ = o.draft_forward(dm, layers, gf, cache, gamma, embed=E, tokens=tok, storage="f32")
    h0 = E[tok]
    want = gf * h0 / np.sqrt(np.mean(h0 ** 2, axis=-1, keepdims=True) + dm.eps)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
    d, _, logits = o.lm_head_argmax(got, E)
    assert np.allclose(logits, np.einsum("bgd,vd->bgv", want[:, 1:], E), rtol=1e-12, atol=1e-10)


def pin_draft_visibility(o):
    # Every block query sees every context row and every block row (no mask):
    # perturbing any one of them changes every query's output.
    rng = _rng(13)
    dm = dims()
    L, B, gamma = 1, 1, 4
    layers = rand_layers(rng, dm, L)
    gf = np.ones(dm.D)
    n = 6
    cache = cache_with(o, L, B, dm.Hkv, dm.d, [n], rng)
    h0 = rng.normal(0, 1, (B, gamma, dm.D))
    base, _ = o.draft_forward(dm, layers, gf, cache, gamma, override=h0, storage="f32")
    for t in (0, n // 2, n - 1):
        c2 = o.OracleCache(L, B, dm.Hkv, dm.d)
        k = cache.k[0][0].copy()
        v = cache.v[0][0].copy()
        k[t] += 0.5
        v[t] -= 0.5
        c2.append(0, 0, k, v)
        out, _ = o.draft_forward(dm, layers, gf, c2, gamma, override=h0, storage="f32")
        assert np.all(np.max(np.abs(out - base), axis=-1) > 1e-6), t
    for i in range(gamma):
        h1 = h0.copy()
        h1[0, i] += 0.5
        out, _ = o.draft_forward(dm, layers, gf, cache, gamma, override=h1, storage="f32")
        others = [r for r in range(gamma) if r != i]
        assert np.all(np.max(np.abs(out[0, others] - base[0, others]), axis=-1) > 1e-6), i


def pin_draft_permutations(o):
    rng = _rng(14)
    dm = dims()
    L, B, gamma = 2, 1, 6
    layers = rand_layers(rng, dm, L)
    gf = np.ones(dm.D)
    n = 9
    cache = cache_with(o, L, B, dm.Hkv, dm.d, [n], rng)
    h0 = rng.normal(0, 1, (B, gamma, dm.D))
    base, _ = o.draft_forward(dm, layers, gf, cache, gamma, override=h0, storage="f32")
    # permuting block rows permutes outputs (no positional encoding)
    p = rng.permutation(gamma)
    out, _ = o.draft_forward(dm, layers, gf, cache, gamma, override=h0[:, p], storage="f32")
    assert np.allclose(out, base[:, p], rtol=1e-12, atol=1e-12)
    # permuting context rows leaves outputs unchanged
    pc = rng.permutation(n)
    c2 = o.OracleCache(L, B, dm.Hkv, dm.d)
    for l in range(L):
        c2.append(l, 0, cache.k[l][0][pc], cache.v[l][0][pc])
    out, _ = o.draft_forward(dm, layers, gf, c2, gamma, override=h0, storage="f32")
    assert np.allclose(out, base, rtol=1e-12, atol=1e-12)


def pin_draft_block_kv_storage(o):
    # The block's own K/V rows are rounded like cache rows: with bf16 storage
    # every returned block key is bf16-exact, and it differs from f32 storage.
    rng = _rng(15)
    dm = dims()
    layers = rand_layers(rng, dm, 1)
    cache = cache_with(o, 1, 1, dm.Hkv, dm.d, [4], rng)
    h0 = rng.normal(0, 1, (1, 3, dm.D))
    a, kv_a = o.draft_forward(dm, layers, np.ones(dm.D), cache, 3, override=h0, storage="bf16")
    b, kv_b = o.draft_forward(dm, layers, np.ones(dm.D), cache, 3, override=h0, storage="f32")
    kb = kv_a[0][0]
    assert np.array_equal(kb, o.to_bf16(kb))
    assert not np.array_equal(kv_a[0][0], kv_b[0][0])


# ---------------------------------------------------------------------------
# argmax / accept
# ---------------------------------------------------------------------------
def pin_argmax_planted(o):
    # Orthonormal block rows z_r = e_r and a planted LM-head row E[v_r] = 5 e_r:
    # the planted token has logit 5, every other logit is small.
    rng = _rng(16)
    B, g, D, V = 2, 5, 12, 50
    rows = B * (g - 1)
    z = np.zeros((B, g, D))
    E = rng.normal(0, 0.1, (V, D))
    planted = rng.choice(V, size=rows, replace=False)
    r = 0
    for b in range(B):
        z[b, 0, D - 1] = 1.0
        for i in range(1, g):
            z[b, i, r] = 1.0
            E[planted[r], r] = 5.0
            r += 1
    d, gap, logits = o.lm_head_argmax(z, E)
    assert np.array_equal(d.reshape(-1), planted)
    assert np.all(gap > 3.0)
    # the anchor row (row 0) is not drafted even if it has the largest logit
    z2 = z.copy()
    z2[:, 0] = 100.0
    d2, _, l2 = o.lm_head_argmax(z2, E)
    assert l2.shape == (B, g - 1, V) and np.array_equal(d2, d)


def pin_argmax_ties(o):
    z = np.zeros((1, 3, 4))
    z[0, 1] = [1, 0, 0, 0]
    z[0, 2] = [0, 1, 0, 0]
    E = np.zeros((6, 4))
    E[2, 0] = 1.0
    E[4, 0] = 1.0          # tie with token 2 -> lowest id wins
    E[5, 1] = 3.0
    E[1, 1] = 2.0
    d, gap, _ = o.lm_head_argmax(z, E)
    assert list(d[0]) == [2, 5]
    assert gap[0, 0] == 0.0 and gap[0, 1] == 1.0


def pin_accept_cases(o):
    n = 6
    d = np.array([[1, 2, 3, 4, 5, 6]] * 5)
    t = np.array([
        [1, 2, 3, 4, 5, 6, 7],      # all match -> tau = n+1, next = bonus
        [9, 2, 3, 4, 5, 6, 7],      # mismatch at 0 -> tau 1
        [1, 2, 9, 4, 5, 6, 7],      # mismatch at 2 -> tau 3 (later matches ignored)
        [1, 2, 3, 4, 5, 9, 7],      # mismatch at n-1 -> tau n
        [1, 9, 9, 9, 9, 9, 9],
    ])
    tau, nxt = o.accept(d, t)
    assert list(tau) == [7, 1, 3, 6, 2]
    assert list(nxt) == [7, 9, 9, 9, 9]
    assert np.all((tau >= 1) & (tau <= n + 1))


def expected_tau(p) -> float:
    """E[tau] = sum_{k=0..n} prod_{j<k} p_j for independent per-position matches."""
    tot, pr = 0.0, 1.0
    for k in range(len(p) + 1):
        tot += pr
        if k < len(p):
            pr *= p[k]
    return tot


def pin_accept_expectation(o):
    # Monte Carlo over seeded blocks against the closed form (3 sigma).
    rng = _rng(17)
    for p in (np.full(15, 0.8), 0.9 - 0.4 * np.arange(15) / 14):
        N, n = 20000, len(p)
        d = rng.integers(0, 1000, (N, n))
        match = rng.random((N, n)) < p
        t = np.where(match, d, (d + rng.integers(1, 1000, (N, n))) % 1000)
        t = np.concatenate([t, rng.integers(0, 1000, (N, 1))], axis=1)
        tau, _ = o.accept(d, t)
        mu = expected_tau(p)
        sd = tau.std() / math.sqrt(N)
        assert abs(tau.mean() - mu) < 3.5 * sd + 1e-9, (tau.mean(), mu)


# ---------------------------------------------------------------------------
# ragged blocks (a block length per sequence)
# ---------------------------------------------------------------------------
def pin_ragged_matches_torch_per_sequence(o):
    # Each sequence of a ragged batch against the library-routine composition of
    # the layers over its own context and its own block length (2, 5, 1+3).
    rng = _rng(40)
    dm = dims()
    L = 2
    layers = rand_layers(rng, dm, L)
    gf = 1 + rng.normal(0, 0.2, dm.D)
    lens = [6, 0, 3]
    gammas = [2, 5, 4]
    cache = cache_with(o, L, 3, dm.Hkv, dm.d, lens, rng)
    h0 = [rng.normal(0, 1, (g, dm.D)) for g in gammas]
    got, kv = o.draft_forward_ragged(dm, layers, gf, cache, gammas, override=h0, storage="f32")
    assert [x.shape for x in got] == [(g, dm.D) for g in gammas]
    for b in range(3):
        ref = _torch_layer_forward(dm, layers, gf, [cache.k[l][b] for l in range(L)],
                                   [cache.v[l][b] for l in range(L)], h0[b])
        assert np.allclose(got[b], ref, rtol=1e-9, atol=1e-9), b
        assert kv[b][0][0].shape == (gammas[b], dm.Hkv, dm.d)


def pin_ragged_uniform_and_independent(o):
    # Equal block lengths reproduce the batched pass exactly; changing one
    # sequence's block length leaves every other sequence's output unchanged.
    rng = _rng(41)
    dm = dims()
    L, B, g = 2, 3, 4
    layers = rand_layers(rng, dm, L)
    gf = 1 + rng.normal(0, 0.2, dm.D)
    cache = cache_with(o, L, B, dm.Hkv, dm.d, [5, 2, 7], rng)
    E = rng.normal(0, 0.3, (20, dm.D))
    tok = rng.integers(0, 20, (B, g))
    uni, _ = o.draft_forward(dm, layers, gf, cache, g, embed=E, tokens=tok, storage="bf16")
    rag, _ = o.draft_forward_ragged(dm, layers, gf, cache, [g] * B, embed=E, tokens=list(tok), storage="bf16")
    for b in range(B):
        assert np.array_equal(rag[b], uni[b])
    tok2 = [tok[0], np.concatenate([tok[1], [3, 9]]), tok[2]]
    rag2, _ = o.draft_forward_ragged(dm, layers, gf, cache, [g, g + 2, g], embed=E, tokens=tok2, storage="bf16")
    assert np.array_equal(rag2[0], rag[0]) and np.array_equal(rag2[2], rag[2])
    assert rag2[1].shape == (g + 2, dm.D) and not np.allclose(rag2[1][:g], rag[1])   # block rows see each other


def pin_ragged_argmax_accept(o):
    # Per-sequence drafts and acceptance with their own lengths, against the
    # batched functions on each sequence and hand-made cases.
    rng = _rng(42)
    D, V = 6, 30
    E = rng.normal(0, 1, (V, D))
    hs = [rng.normal(0, 1, (g, D)) for g in (2, 6, 4)]
    d, gaps, z = o.lm_head_argmax_ragged(hs, E)
    assert [x.shape for x in d] == [(1,), (5,), (3,)]
    for b, h in enumerate(hs):
        d1, _, z1 = o.lm_head_argmax(h[None], E)
        assert np.array_equal(d[b], d1[0]) and np.allclose(z[b], z1[0])
    drafts = [np.array([4]), np.array([1, 2, 3, 4, 5]), np.array([7, 8, 9])]
    targets = [np.array([4, 11]), np.array([1, 2, 0, 4, 5, 6]), np.array([6, 8, 9, 2])]
    tau, nxt = o.accept_ragged(drafts, targets)
    assert list(tau) == [2, 3, 1] and list(nxt) == [11, 0, 6]


# ---------------------------------------------------------------------------
# anchored blocks (the training-style forward)
# ---------------------------------------------------------------------------
def pin_blocks_match_torch_on_prefix(o):
    # Each block against the torch composition of the layers over its own
    # sequence's context rows [0, anchor) and its own rows only.
    rng = _rng(50)
    dm = dims()
    L, g = 2, 4
    layers = rand_layers(rng, dm, L)
    gf = 1 + rng.normal(0, 0.2, dm.D)
    cache = cache_with(o, L, 2, dm.Hkv, dm.d, [9, 6], rng)
    blocks = [(0, 0), (0, 4), (1, 6), (0, 9)]
    h0 = rng.normal(0, 1, (len(blocks), g, dm.D))
    got, kv = o.draft_forward_blocks(dm, layers, gf, cache, blocks, g, override=h0, storage="f32")
    assert got.shape == (4, g, dm.D) and len(kv) == 4
    for k, (sq, a) in enumerate(blocks):
        ref = _torch_layer_forward(dm, layers, gf, [cache.k[l][sq][:a] for l in range(L)],
                                   [cache.v[l][sq][:a] for l in range(L)], h0[k])
        assert np.allclose(got[k], ref, rtol=1e-9, atol=1e-9), k


def pin_blocks_visibility(o):
    # A block anchored at a: context rows before a change it, rows at or after a
    # do not, nor does any other block's input; anchoring at the full length is
    # the inference pass.
    rng = _rng(51)
    dm = dims()
    L, g = 2, 3
    layers = rand_layers(rng, dm, L)
    gf = 1 + rng.normal(0, 0.2, dm.D)
    cache = cache_with(o, L, 1, dm.Hkv, dm.d, [8], rng)
    blocks = [(0, 5), (0, 2)]
    h0 = rng.normal(0, 1, (2, g, dm.D))
    base, _ = o.draft_forward_blocks(dm, layers, gf, cache, blocks, g, override=h0, storage="f32")
    for row, changes in ((4, True), (0, True), (5, False), (7, False)):
        c2 = cache_with(o, L, 1, dm.Hkv, dm.d, [0], rng)
        for l in range(L):
            k = cache.k[l][0].copy()
            v = cache.v[l][0].copy()
            k[row] += 0.5
            v[row] -= 0.5
            c2.append(l, 0, k, v)
        got, _ = o.draft_forward_blocks(dm, layers, gf, c2, blocks, g, override=h0, storage="f32")
        assert (not np.allclose(got[0], base[0])) == changes, row
        assert np.all(np.any(np.abs(got[0] - base[0]) > 1e-12, axis=1)) == changes
        assert np.array_equal(got[1], base[1]) == (row >= 2)
    h1 = h0.copy()
    h1[1] += 1.0
    got, _ = o.draft_forward_blocks(dm, layers, gf, cache, blocks, g, override=h1, storage="f32")
    assert np.array_equal(got[0], base[0])
    full, _ = o.draft_forward_blocks(dm, layers, gf, cache, [(0, 8)], g, override=h0[:1], storage="f32")
    inf, _ = o.draft_forward(dm, layers, gf, cache, g, override=h0[:1], storage="f32")
    assert np.array_equal(full, inf)


# ---------------------------------------------------------------------------
# sampled drafting / lossless verification
# ---------------------------------------------------------------------------
def _softmax(x, T=1.0):
    from scipy.special import softmax
    return softmax(np.asarray(x, dtype=F64) / T, axis=-1)


def _freq_ok(samples, probs, n_sigma=5.0):
    """Empirical category frequencies of integer samples within n_sigma binomial
    standard errors of probs (and no sample outside the support)."""
    samples = np.asarray(samples).reshape(-1)
    N, V = samples.size, len(probs)
    assert N > 0
    cnt = np.bincount(samples, minlength=V)
    assert cnt.size == V, "sample outside the vocabulary"
    f = cnt / N
    se = np.sqrt(np.maximum(probs * (1 - probs), 1e-12) / N)
    return bool(np.all(np.abs(f - probs) <= n_sigma * se + 1e-12)), f


def pin_gumbel_pick_distribution(o):
    # The Gumbel-max draw follows softmax(logw); a -inf weight is never drawn;
    # for two categories P(0) = sigmoid(logw0 - logw1) (closed form).
    rng = _rng(30)
    N = 200000
    logw = np.array([0.3, -1.2, 1.1, -np.inf, 0.0])
    u = rng.random((N, 5))
    idx, gap = o.gumbel_pick(np.broadcast_to(logw, (N, 5)), u)
    ok, f = _freq_ok(idx, _softmax(np.where(np.isinf(logw), -1e300, logw)))
    assert ok, f
    assert not np.any(idx == 3)
    assert np.all(gap >= 0)
    lw2 = np.array([0.7, -0.4])
    idx2, _ = o.gumbel_pick(np.broadcast_to(lw2, (N, 2)), u[:, :2])
    p0 = 1.0 / (1.0 + math.exp(-(lw2[0] - lw2[1])))
    assert abs(np.mean(idx2 == 0) - p0) < 5 * math.sqrt(p0 * (1 - p0) / N)
    # exact ties (equal weights, equal uniforms) go to the lowest index
    t_idx, t_gap = o.gumbel_pick(np.zeros((1, 4)), np.full((1, 4), 0.5))
    assert t_idx[0] == 0 and t_gap[0] == 0.0


def pin_logsumexp_library(o):
    from scipy.special import logsumexp
    rng = _rng(31)
    z = rng.normal(0, 3.0, (3, 4, 257))
    for T in (1.0, 0.6, 2.5):
        assert np.allclose(o.logsumexp_t(z, T), logsumexp(z / T, axis=-1), rtol=0, atol=1e-12)
        ref = torch.log_softmax(torch.from_numpy(z / T), dim=-1).numpy()
        assert np.allclose(o.log_softmax_t(z, T), ref, rtol=0, atol=1e-12)


def pin_sample_drafts_distribution(o):
    # Block rows e_1, e_2 against an LM head whose column i holds the logits of
    # row i: the drafts at mask row i follow softmax(column_i / T); the anchor
    # row is not drafted; logits and log-normalisers match the closed forms.
    from scipy.special import logsumexp
    rng = _rng(32)
    V, D, N, T = 6, 3, 60000, 0.7
    E = rng.normal(0, 1.2, (V, D))
    h = np.zeros((N, 3, D))
    h[:, 0, 0] = 1.0       # anchor row: never drafted
    h[:, 1, 1] = 1.0
    h[:, 2, 2] = 1.0
    u = rng.random((N, 2, V))
    d, z, lse, gap = o.sample_drafts(h, E, T, u)
    assert d.shape == (N, 2) and z.shape == (N, 2, V)
    assert np.allclose(z[0, 0], E[:, 1]) and np.allclose(z[0, 1], E[:, 2])
    assert np.allclose(lse[0], logsumexp(E[:, 1:3].T / T, axis=-1), atol=1e-12)
    for i in (1, 2):
        ok, f = _freq_ok(d[:, i - 1], _softmax(E[:, i], T))
        assert ok, (i, f)
    # the two positions are drawn independently (uniforms of their own)
    joint = np.mean((d[:, 0] == 0) & (d[:, 1] == 0))
    pa, pb = _softmax(E[:, 1], T)[0], _softmax(E[:, 2], T)[0]
    assert abs(joint - pa * pb) < 5 * math.sqrt(pa * pb / N)
    # temperature -> 0 with well separated logits: the draw is the greedy argmax
    h1 = rng.normal(0, 1, (4, 5, D))
    E1 = rng.normal(0, 1, (V, D))
    g_d, g_gap, _ = o.lm_head_argmax(h1, E1)
    s_d, _, _, _ = o.sample_drafts(h1, E1, 1e-6, rng.uniform(0.01, 0.99, (4, 4, V)))
    keep = g_gap > 1e-3
    assert np.array_equal(s_d[keep], g_d[keep])


def _committed(draft, tau, nxt):
    """Committed tokens of each block: d_0..d_{tau-2} then the emitted token."""
    out = []
    for b in range(len(tau)):
        out.append(list(draft[b, :tau[b] - 1]) + [int(nxt[b])])
    return out


def pin_sample_accept_lossless(o):
    # Losslessness ([GL] "비용 구조의 차이가 만드는 성능 격차"): with drafts drawn
    # from q_j, the token committed at every position follows the target's p_j,
    # and position k is reached with probability prod_{j<k} sum_v min(p_j, q_j).
    rng = _rng(33)
    V, n, T, N = 4, 3, 0.8, 40000
    z = rng.normal(0, 1.5, (n, V))
    t = rng.normal(0, 1.5, (n + 1, V))
    q, p = _softmax(z, T), _softmax(t, T)
    d = np.stack([rng.choice(V, size=N, p=q[j]) for j in range(n)], axis=1)
    au = rng.random((N, n))
    ru = rng.random((N, V))
    tau, nxt, info = o.sample_accept(d, np.broadcast_to(z, (N, n, V)), np.broadcast_to(t, (N, n + 1, V)),
                                     T, au, ru)
    assert np.all((tau >= 1) & (tau <= n + 1))
    com = _committed(d, tau, nxt)
    for k in range(n + 1):
        toks = np.array([c[k] for c in com if len(c) > k])
        ok, f = _freq_ok(toks, p[k])
        assert ok, (k, f, p[k])
    beta = np.minimum(p[:n], q).sum(axis=1)
    reach = 1.0
    for k in range(n + 1):
        emp = np.mean(tau >= k + 1)
        assert abs(emp - reach) <= 5 * math.sqrt(max(reach * (1 - reach), 1e-12) / N) + 1e-12, (k, emp, reach)
        if k < n:
            reach *= beta[k]


def pin_sample_accept_cases(o):
    V, n, T = 8, 3, 1.0
    rng = _rng(34)
    z = rng.normal(0, 1, (1, n, V))
    d = np.array([[2, 5, 1]])
    ru = rng.random((1, V))
    # identical draft and target distributions: everything is accepted (u < 1)
    t = np.concatenate([z, np.zeros((1, 1, V))], axis=1)
    t[0, n, 6] = 60.0                                   # bonus row: one-hot on 6
    tau, nxt, _ = o.sample_accept(d, z, t, T, np.full((1, n), 0.999), ru)
    assert tau[0] == n + 1 and nxt[0] == 6
    # the target gives draft 0 (almost) no mass and peaks on token 7: rejected at
    # 0, and the residual max(0, p - q) is (almost) all on token 7
    t2 = t.copy()
    t2[0, 0] = 0.0
    t2[0, 0, 7] = 60.0
    tau, nxt, info = o.sample_accept(d, z, t2, T, np.full((1, n), 1e-9), ru)
    assert tau[0] == 1 and nxt[0] == 7 and info["m"][0] == 0
    # p(d_j) > q(d_j) is accepted whatever the uniform; rejection at 1 from a
    # target that puts no mass on d_1 = 5
    t3 = t.copy()
    t3[0, 0, 2] = z[0, 0, 2] + 3.0
    t3[0, 1, 5] = -60.0
    tau, nxt, info = o.sample_accept(d, z, t3, T, np.array([[0.999999, 1e-9, 0.5]]), ru)
    assert tau[0] == 2 and nxt[0] != 5 and info["log_ratio"][0, 0] > 0
    # a rejection with p == q (only a uniform of 1 rejects) leaves an empty
    # residual: the draw then comes from p_m itself
    t4 = t.copy()
    t4[0, 1] = z[0, 1]
    z4 = z.copy()
    z4[0, 1, 3] = 60.0
    t4[0, 1, 3] = 60.0
    tau, nxt, info = o.sample_accept(d, z4, t4, T, np.array([[0.5, 1.0, 0.5]]), ru)
    assert tau[0] == 2 and nxt[0] == 3 and info["resid_empty"][0]


# ---------------------------------------------------------------------------
# the target side: tapped layers and the causal verify forward
# ---------------------------------------------------------------------------
GOLD_TAPS = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden", "tap_layers.txt")


def pin_tap_layers_golden(o):
    # hand-worked indices for several target depths (tests/golden/tap_layers.txt)
    for line in open(GOLD_TAPS, encoding="utf-8"):
        line = line.split("#")[0].split()
        if line:
            L_t, want = int(line[0]), [int(x) for x in line[1:]]
            assert list(o.tap_layers(L_t)) == want, (L_t, o.tap_layers(L_t), want)
    # the rule's shape at every depth: second layer first, third-from-last
    # last, strictly increasing, spacings that differ by at most one
    for L_t in range(8, 101):
        t = np.asarray(o.tap_layers(L_t))
        gaps = np.diff(t)
        assert t[0] == 1 and t[-1] == L_t - 3 and len(t) == 5, (L_t, t)
        assert gaps.min() >= 1 and gaps.max() - gaps.min() <= 1, (L_t, t)


def _torch_target_forward(dm, layers, g_final, ctx_k, ctx_v, h0, taps):
    """Library-routine composition (float64 CPU) of a causal target forward:
    SDPA over [context; block] with an explicit boolean mask (block row i sees
    every context row and block rows 0..i); f32 storage of the block K/V and of
    the tapped states emulated by float32 round trips.  Returns (normed final
    states, {layer: residual stream after it})."""
    D, Hq, Hkv, d, F, eps = dm.D, dm.Hq, dm.Hkv, dm.d, dm.F, dm.eps
    G = Hq // Hkv
    h = torch.from_numpy(h0.copy())
    g_ = h.shape[0]
    n_ctx = ctx_k[0].shape[0]
    mask = torch.ones(g_, n_ctx + g_, dtype=torch.bool)
    mask[:, n_ctx:] = torch.tril(torch.ones(g_, g_, dtype=torch.bool))

    def norm(x, g):
        m = torch.nn.RMSNorm(D, eps=eps, dtype=torch.float64)
        with torch.no_grad():
            m.weight.copy_(torch.from_numpy(np.asarray(g, dtype=F64)))
            return m(x)

    kept = {}
    with torch.no_grad():
        for l, w in enumerate(layers):
            a = norm(h, w["g_attn"])
            wq = torch.from_numpy(w["w_qkv"][: Hq * d])
            wk = torch.from_numpy(w["w_qkv"][Hq * d:(Hq + Hkv) * d])
            wv = torch.from_numpy(w["w_qkv"][(Hq + Hkv) * d:])
            q = torch.nn.functional.linear(a, wq).reshape(g_, Hq, d).permute(1, 0, 2)
            kb = torch.nn.functional.linear(a, wk).float().double().reshape(g_, Hkv, d)
            vb = torch.nn.functional.linear(a, wv).float().double().reshape(g_, Hkv, d)
            K = torch.cat([torch.from_numpy(ctx_k[l]), kb], 0).permute(1, 0, 2).repeat_interleave(G, 0)
            Vv = torch.cat([torch.from_numpy(ctx_v[l]), vb], 0).permute(1, 0, 2).repeat_interleave(G, 0)
            att = torch.nn.functional.scaled_dot_product_attention(q, K, Vv, attn_mask=mask)
            att = att.permute(1, 0, 2).reshape(g_, Hq * d)
            h = h + torch.nn.functional.linear(att, torch.from_numpy(w["w_o"]))
            f = norm(h, w["g_ffn"])
            gu = torch.nn.functional.linear(f, torch.from_numpy(w["w_gateup"]))
            s = torch.nn.functional.silu(gu[:, :F]) * gu[:, F:]
            h = h + torch.nn.functional.linear(s, torch.from_numpy(w["w_down"]))
            if l in taps:
                kept[l] = h.float().double().numpy()
        return norm(h, g_final).numpy(), kept


def _target_setup(seed, L=3, B=2, lens=(6, 0), V=40):
    rng = _rng(seed)
    dm = dims()
    layers = rand_layers(rng, dm, L)
    gf = 1 + rng.normal(0, 0.2, dm.D)
    E = rng.normal(0, 1, (V, dm.D))
    return rng, dm, layers, gf, E


def pin_target_torch_composition(o):
    rng, dm, layers, gf, E = _target_setup(31)
    lens, gamma, taps = [6, 0], 5, [0, 2]
    cache = cache_with(o, len(layers), 2, dm.Hkv, dm.d, lens, rng)
    tok = rng.integers(0, E.shape[0], (2, gamma))
    res = o.target_verify(dm, layers, gf, E, E, cache, tok, taps, storage="f32", tap_storage="f32")
    for b in range(2):
        zf, kept = _torch_target_forward(dm, layers, gf, [cache.k[l][b] for l in range(len(layers))],
                                         [cache.v[l][b] for l in range(len(layers))], E[tok[b]], taps)
        ref_logits = zf @ E.T
        assert np.allclose(res["logits"][b], ref_logits, rtol=1e-9, atol=1e-9), b
        assert np.array_equal(res["tokens"][b], np.argmax(ref_logits, axis=-1)), b
        for k, l in enumerate(taps):
            assert np.allclose(res["taps"][k][b], kept[l], rtol=1e-9, atol=1e-9), (b, l)


def pin_target_prefix_consistency(o):
    # causal attention: a block row depends only on the rows before it, so
    # verifying the first i+1 tokens alone gives row i's outputs exactly
    rng, dm, layers, gf, E = _target_setup(32)
    lens, gamma, taps = [4, 0], 6, [1]
    cache = cache_with(o, len(layers), 2, dm.Hkv, dm.d, lens, rng)
    tok = rng.integers(0, E.shape[0], (2, gamma))
    full = o.target_verify(dm, layers, gf, E, E, cache, tok, taps, storage="f32", tap_storage="f32")
    for i in range(gamma):
        part = o.target_verify(dm, layers, gf, E, E, cache, tok[:, :i + 1], taps, storage="f32",
                               tap_storage="f32")
        assert np.allclose(part["logits"][:, i], full["logits"][:, i], rtol=1e-10, atol=1e-10), i
        assert np.allclose(part["taps"][0][:, i], full["taps"][0][:, i], rtol=1e-10, atol=1e-10), i
    # and a later token never moves an earlier row, while it does move its own
    tok2 = tok.copy()
    tok2[:, 3] = (tok2[:, 3] + 1) % E.shape[0]
    alt = o.target_verify(dm, layers, gf, E, E, cache, tok2, taps, storage="f32", tap_storage="f32")
    assert np.array_equal(alt["logits"][:, :3], full["logits"][:, :3])
    assert not np.allclose(alt["logits"][:, 3], full["logits"][:, 3])


def pin_target_greedy_lossless(o):
    # Greedy speculative decoding is lossless: if the drafts are the target's
    # own greedy continuation, one parallel verify reproduces it and accepts
    # every draft; a wrong draft at position m stops acceptance there and the
    # next anchor is the target's own token.  The continuation comes from
    # autoregressive decoding (one row per call, its K/V appended each time).
    rng, dm, layers, gf, E = _target_setup(33, B=1, lens=(5,))
    L, n = len(layers), 6
    cache = cache_with(o, L, 1, dm.Hkv, dm.d, [5], rng)
    ar = o.OracleCache(L, 1, dm.Hkv, dm.d)
    for l in range(L):
        ar.append(l, 0, cache.k[l][0], cache.v[l][0])
    seq = [int(rng.integers(0, E.shape[0]))]
    for _ in range(n + 1):
        r = o.target_verify(dm, layers, gf, E, E, ar, np.array([[seq[-1]]]), [], storage="f32")
        for l, (kb, vb) in enumerate(r["block_kv"]):
            ar.append(l, 0, kb[0], vb[0])
        seq.append(int(r["tokens"][0, 0]))
    anchor, cont = seq[0], seq[1:]
    res = o.target_verify(dm, layers, gf, E, E, cache, np.array([[anchor] + cont[:n]]), [], storage="f32")
    assert list(res["tokens"][0]) == cont, (list(res["tokens"][0]), cont)
    tau, nxt = o.accept(np.array([cont[:n]]), res["tokens"])
    assert tau[0] == n + 1 and nxt[0] == cont[n]
    for m in (0, 3):
        dr = list(cont[:n])
        dr[m] = (dr[m] + 1) % E.shape[0]
        res = o.target_verify(dm, layers, gf, E, E, cache, np.array([[anchor] + dr]), [], storage="f32")
        assert list(res["tokens"][0][:m + 1]) == cont[:m + 1]
        tau, nxt = o.accept(np.array([dr]), res["tokens"])
        assert tau[0] == m + 1 and nxt[0] == cont[m], (m, tau, nxt)


def pin_target_zero_branches(o):
    # W_O = 0 and W_down = 0: every layer passes the residual stream through,
    # so every tapped state is the token embedding itself and the logits are
    # E . RMSNorm(E[token]; g_final), in closed form
    rng, dm, layers, gf, E = _target_setup(34)
    for w in layers:
        w["w_o"] = np.zeros_like(w["w_o"])
        w["w_down"] = np.zeros_like(w["w_down"])
    cache = cache_with(o, len(layers), 2, dm.Hkv, dm.d, [3, 2], rng)
    tok = rng.integers(0, E.shape[0], (2, 4))
    res = o.target_verify(dm, layers, gf, E, E, cache, tok, [0, 1, 2], storage="f32", tap_storage="f32")
    for t in res["taps"]:
        assert np.array_equal(t, E[tok].astype(np.float32).astype(F64))
    x = E[tok]
    z = gf * x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + dm.eps)
    assert np.allclose(res["logits"], z @ E.T, rtol=1e-12, atol=1e-12)
    # the argmax covers every row, the anchor's included: plant the best token
    E2 = E.copy()
    E2[7] = 50.0 * z[0, 0] / np.linalg.norm(z[0, 0])
    res2 = o.target_verify(dm, layers, gf, E, E2, cache, tok, [], storage="f32")
    assert res2["tokens"][0, 0] == 7 and res2["gap"][0, 0] > 0


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
