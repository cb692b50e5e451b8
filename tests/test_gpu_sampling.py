"""GPU parity of sampled drafting and lossless verification against the oracle.

Both sides get the same seeded inputs (h_final rows, LM head, uniforms, target
logits) and compute independently; nothing the GPU produces is fed to the
oracle.  Comparisons:
  * logits: the LM-head tolerances of the greedy path (bf16: max-abs 2e-2 and
    relative 1e-2; fp32: 1e-4 and 1e-5);
  * log-normalisers log sum exp(z / T): within (logits max-abs error) / T + 1e-4;
  * draft ids: equal on every row whose oracle Gumbel-key gap (best minus
    runner-up of z / T + G(u)) is at least 1e-3 * max(1, 1 / T): the fp32
    keys then cannot swap order;
  * tau and the emitted token: equal for every sequence whose oracle decisions
    have margins the fp32 kernels resolve: |log u_j - log(p_j(d_j)/q_j(d_j))|
    >= 1e-4 at every decided position j <= m, and an emitted-token key gap
    >= 2e-3.  Excluded sequences are counted and must stay rare.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from block_diffusion_drafter_ctx_amd import binding as B
from block_diffusion_drafter_ctx_amd.runtime import dims_of, upload
from dflash_inputs import BATCH16_RAGGED, QWEN3_8B_N2048, TINY_F32, Inputs, build_target_logits_np, shrink
from oracle import dflash_oracle as O
from tests.parity_util import close, log

pytestmark = pytest.mark.gpu

LOGIT_STD = 1.28          # spread of the drafter's logits at D = 4096 (0.02 * sqrt(4096))
ACCEPT_MARGIN = 1e-4
EMIT_GAP = 2e-3


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


class Head:
    """The LM head of one workload on both sides, plus a workspace."""

    def __init__(self, cfg, gamma):
        self.cfg = cfg
        self.inp = Inputs(cfg)
        E = self.inp.embed()
        self.E_dev = upload(E, cfg)
        self.E64 = E.astype(np.float64)
        self.dims = dims_of(cfg)
        self.w = B.Weights(lm_head=self.E_dev.data_ptr())
        self.ws_bytes = B.workspace_size(self.dims, cfg.B, gamma, 1)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device="cuda")

    def sample(self, h, gamma, T, u, with_lse=True):
        Bn, n, V = self.cfg.B, gamma - 1, self.cfg.V
        d = torch.full((Bn, n), -7, dtype=torch.int32, device="cuda")
        z = torch.full((Bn, n, V), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((Bn, n), float("nan"), dtype=torch.float32, device="cuda") if with_lse else None
        B.sample_drafts(self.dims, self.w, h.data_ptr(), Bn, gamma, T, u.data_ptr(), d.data_ptr(), z.data_ptr(),
                        0 if lse is None else lse.data_ptr(), self.ws.data_ptr(), self.ws_bytes, _stream())
        return d, z, lse


def accept_gpu(dims, Bn, gamma, T, d, z, t, au, ru, lse=None):
    need = B.workspace_size(dims, Bn, gamma, 1)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    tau = torch.full((Bn,), -1, dtype=torch.int32, device="cuda")
    nxt = torch.full((Bn,), -1, dtype=torch.int32, device="cuda")
    B.sample_accept(dims, Bn, gamma, T, d.data_ptr(), z.data_ptr(), 0 if lse is None else lse.data_ptr(),
                    t.data_ptr(), au.data_ptr(), ru.data_ptr(), tau.data_ptr(), nxt.data_ptr(), ws.data_ptr(),
                    need, _stream())
    torch.cuda.synchronize()
    return tau.cpu().numpy(), nxt.cpu().numpy()


def check_drafts(tag, cfg, T, d_g, z_g, l_g, d_o, z_o, l_o, gap_o):
    z_g = z_g.cpu().numpy()
    err, rel = close(z_g, z_o, cfg.dtype, f"{tag} logits")
    if l_g is not None:
        e_l = float(np.max(np.abs(l_g.cpu().numpy() - l_o)))
        assert e_l <= err / T + 1e-4, f"{tag} lse max-abs {e_l:.3e} (logits err {err:.3e}, T {T})"
    else:
        e_l = float("nan")
    d_g = d_g.cpu().numpy()
    assert d_g.min() >= 0 and d_g.max() < cfg.V
    key_min = 1e-3 * max(1.0, 1.0 / T)
    keep = gap_o >= key_min
    bad = np.argwhere((d_g != d_o) & keep)
    assert bad.size == 0, f"{tag}: draft differs at {bad[:8].tolist()} (oracle key gaps {gap_o[tuple(bad[:8].T)]})"
    excl = int((~keep).sum())
    assert excl <= max(1, d_o.size // 20), f"{tag}: {excl} of {d_o.size} rows have near-tied keys"
    log(f"{tag}: logits max-abs {err:.2e} rel {rel:.2e}; lse max-abs {e_l:.2e}; drafts agree "
        f"({excl} near-tie rows of {d_o.size} excluded); min key gap {gap_o.min():.2e}")
    return d_g


def check_accept(tag, tau_g, nxt_g, d, z, t, T, au, ru):
    tau_o, nxt_o, info = O.sample_accept(d, z, t, T, au, ru)
    Bn, n = d.shape
    amarg = np.abs(np.log(np.asarray(au, dtype=np.float64)) - info["log_ratio"])
    near = np.zeros(Bn, dtype=bool)
    for b in range(Bn):
        jm = min(int(info["m"][b]), n - 1)
        near[b] = bool(np.any(amarg[b, :jm + 1] < ACCEPT_MARGIN)) or info["key_gap"][b] < EMIT_GAP
    ok = ~near
    assert np.array_equal(tau_g[ok], tau_o[ok]), f"{tag}: tau {tau_g[ok][:16]} vs oracle {tau_o[ok][:16]}"
    assert np.array_equal(nxt_g[ok], nxt_o[ok]), f"{tag}: next {nxt_g[ok][:16]} vs oracle {nxt_o[ok][:16]}"
    assert np.all((tau_g >= 1) & (tau_g <= n + 1)) and np.all((nxt_g >= 0) & (nxt_g < z.shape[-1]))
    assert int(near.sum()) <= max(1, Bn // 10), f"{tag}: {int(near.sum())} of {Bn} sequences near a decision edge"
    log(f"{tag}: tau {tau_o.tolist()[:16]} agree ({int(near.sum())} of {Bn} near-edge sequences excluded; "
        f"{int(info['resid_empty'].sum())} empty residuals)")
    return tau_o, nxt_o, info


# ------------------------------------------------------------------ drafting
DRAFT_CASES = [
    # name, workload, overrides, gamma, T
    ("f32_tiny_T1", TINY_F32, dict(), 16, 1.0),
    ("f32_tiny_b3_g9_T06", TINY_F32, dict(B=3), 9, 0.6),
    ("bf16_rk_m15", QWEN3_8B_N2048, dict(D=2048, V=20000, B=1), 16, 1.0),
    ("bf16_rk_m16_ragged_v", QWEN3_8B_N2048, dict(D=2048, V=20001, B=1), 17, 0.8),
    ("bf16_rk_m1", QWEN3_8B_N2048, dict(D=2048, V=20000, B=1), 2, 1.3),
    ("bf16_rk_chunks_m30", QWEN3_8B_N2048, dict(D=2048, V=20001, B=2), 16, 1.0),
    ("bf16_stream_m60", QWEN3_8B_N2048, dict(D=2048, V=20000, B=4), 16, 1.0),
    ("bf16_tiled_m75_ragged_v", QWEN3_8B_N2048, dict(D=2048, V=20001, B=5), 16, 1.0),
    ("bf16_small_v", QWEN3_8B_N2048, dict(D=256, V=1000, B=2), 16, 0.5),
    ("bf16_rk_hot_T", QWEN3_8B_N2048, dict(D=2048, V=20000, B=1), 16, 25.0),
    ("bf16_rk_cold_T", QWEN3_8B_N2048, dict(D=2048, V=20000, B=1), 16, 0.05),
]


@pytest.mark.parametrize("name,base,kw,gamma,T", DRAFT_CASES, ids=[c[0] for c in DRAFT_CASES])
def test_sample_drafts(name, base, kw, gamma, T):
    cfg = shrink(base, **kw) if kw else base
    log(f"sample_drafts {name}: B={cfg.B} gamma={gamma} D={cfg.D} V={cfg.V} T={T} {cfg.dtype}")
    head = Head(cfg, gamma)
    h = head.inp.final_states(gamma)
    u, _, _ = head.inp.sample_uniforms(0, gamma)
    d_g, z_g, l_g = head.sample(_dev(h), gamma, T, _dev(u))
    d_lean, z_lean, _ = head.sample(_dev(h), gamma, T, _dev(u), with_lse=False)
    torch.cuda.synchronize()
    assert torch.equal(d_g, d_lean) and torch.equal(z_g, z_lean), "results depend on whether lse is requested"
    d_o, z_o, l_o, gap_o = O.sample_drafts(h, head.E64, T, u)
    check_drafts(name, cfg, T, d_g, z_g, l_g, d_o, z_o, l_o, gap_o)


@pytest.mark.parametrize("cfg", [QWEN3_8B_N2048, BATCH16_RAGGED], ids=lambda c: c.name)
def test_sample_drafts_full(cfg):
    """The full-size LM head (V = 151936, D = 4096): one sequence (the register-K
    kernel with the sampling epilogue, as timed) and 16 sequences (tiled GEMM,
    then the row-statistics pass)."""
    gamma, T = 16, 1.0
    log(f"sample_drafts full config {cfg.name}: B={cfg.B}")
    head = Head(cfg, gamma)
    h = head.inp.final_states(gamma)
    u, _, _ = head.inp.sample_uniforms(0, gamma)
    d_g, z_g, l_g = head.sample(_dev(h), gamma, T, _dev(u))
    torch.cuda.synchronize()
    d_o, z_o, l_o, gap_o = O.sample_drafts(h, head.E64, T, u)
    check_drafts(cfg.name, cfg, T, d_g, z_g, l_g, d_o, z_o, l_o, gap_o)
    # the drafts are a sample, not the argmax: most rows differ from it
    greedy = np.argmax(z_o, axis=-1)
    assert np.mean(greedy == d_o) < 0.5


def test_sample_drafts_deterministic():
    cfg = shrink(QWEN3_8B_N2048, D=2048, V=20000, B=1)
    head = Head(cfg, 16)
    h = _dev(head.inp.final_states(16))
    u = _dev(head.inp.sample_uniforms(0, 16)[0])
    a = head.sample(h, 16, 1.0, u)
    b = head.sample(h, 16, 1.0, u)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ------------------------------------------------------------------ verification
ACCEPT_CASES = [
    # name, V, B, gamma, T, pass the draft log-normalisers
    ("v1024_b3_T1", 1024, 3, 16, 1.0, False),
    ("v1024_b3_T07_lse", 1024, 3, 16, 0.7, True),
    ("v20001_ragged_b2_g9", 20001, 2, 9, 1.0, False),
    ("v5000_g2", 5000, 4, 2, 1.0, True),
    ("v1024_b64", 1024, 64, 16, 1.0, False),
    ("v151936_b1_g16", 151936, 1, 16, 1.0, True),
    ("v151936_b16_g33", 151936, 16, 33, 1.0, False),
    ("v151936_b4_g16_T2", 151936, 4, 16, 2.0, True),
]


def _accept_inputs(cfg, gamma, T, it=0):
    inp = Inputs(cfg)
    z = inp.synthetic_logits(it, gamma, LOGIT_STD)
    t = build_target_logits_np(z, inp.target_noise(it, gamma))
    d = inp.random_ids(it, gamma)
    _, au, ru = inp.sample_uniforms(it, gamma)
    return z, t, d, au, ru


@pytest.mark.parametrize("name,V,Bn,gamma,T,with_lse", ACCEPT_CASES, ids=[c[0] for c in ACCEPT_CASES])
def test_sample_accept(name, V, Bn, gamma, T, with_lse):
    cfg = shrink(QWEN3_8B_N2048, V=V, B=Bn)
    log(f"sample_accept {name}: B={Bn} gamma={gamma} V={V} T={T} lse={'given' if with_lse else 'computed'}")
    z, t, d, au, ru = _accept_inputs(cfg, gamma, T)
    z_d = _dev(z)
    lse = torch.logsumexp(z_d / T, dim=-1) if with_lse else None
    tau, nxt = accept_gpu(dims_of(cfg), Bn, gamma, T, _dev(d), z_d, _dev(t), _dev(au), _dev(ru), lse)
    tau_o, _, _ = check_accept(name, tau, nxt, d, z, t, T, au, ru)
    if Bn >= 16:
        # random drafts against the 0.8-overlap recipe: a spread of acceptance lengths
        assert 1 < len(set(tau_o.tolist()))


def test_sample_accept_edges():
    V, Bn, gamma, T = 4096, 6, 12, 1.0
    cfg = shrink(QWEN3_8B_N2048, V=V, B=Bn)
    dims = dims_of(cfg)
    z, t, d, au, ru = _accept_inputs(cfg, gamma, T, it=3)
    n = gamma - 1
    # identical draft and target rows: every draft is kept (the ratio is exactly 1)
    t_same = t.copy()
    t_same[:, :n] = z
    tau, nxt = accept_gpu(dims, Bn, gamma, T, _dev(d), _dev(z), _dev(t_same), _dev(au), _dev(ru))
    assert np.all(tau == n + 1)
    check_accept("edges/all-kept", tau, nxt, d, z, t_same, T, au, ru)
    # a uniform of 1 rejects even at ratio 1; the residual is then empty and the
    # emitted token is a draw from p_m itself
    au1 = au.copy()
    au1[:, 4] = 1.0
    tau, nxt = accept_gpu(dims, Bn, gamma, T, _dev(d), _dev(z), _dev(t_same), _dev(au1), _dev(ru))
    assert np.all(tau == 5)
    # both sides decide position 4 exactly (u = 1 against a ratio of exactly 1),
    # so only the emitted draw's own margin matters here
    tau_o, nxt_o, info = O.sample_accept(d, z, t_same, T, au1, ru)
    assert np.all(tau_o == 5) and np.all(info["resid_empty"])
    keep = info["key_gap"] >= EMIT_GAP
    assert keep.sum() >= Bn - 1 and np.array_equal(nxt[keep], nxt_o[keep])
    # the target puts (almost) all mass on one token: rejected at 0 unless the
    # draft is that token, and the emitted token is that token
    t_peak = t.copy()
    peak = (d[:, 0] + 17) % V
    t_peak[np.arange(Bn), 0, peak] = 80.0
    tau, nxt = accept_gpu(dims, Bn, gamma, T, _dev(d), _dev(z), _dev(t_peak), _dev(au), _dev(ru))
    assert np.all(tau == 1) and np.array_equal(nxt, peak)
    check_accept("edges/peaked-target", tau, nxt, d, z, t_peak, T, au, ru)
    # draft ids outside [0, V) are clamped
    d_out = d.copy()
    d_out[:, 0] = -5
    d_out[:, 1] = V + 3
    d_cl = np.clip(d_out, 0, V - 1).astype(np.int32)
    a = accept_gpu(dims, Bn, gamma, T, _dev(d_out), _dev(z), _dev(t), _dev(au), _dev(ru))
    b = accept_gpu(dims, Bn, gamma, T, _dev(d_cl), _dev(z), _dev(t), _dev(au), _dev(ru))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------------------ chained
def test_sample_chain_qwen3_8b_n2048():
    """Draft, then verify, at the full Qwen3-8B-shaped LM head.  The drafts are
    compared with the oracle's; the verify then runs on identical inputs on
    both sides (the oracle's drafts and draft logits, the target logits built
    from those logits and the seeded noise), so it is always compared.  The
    GPU's own chain (its drafts, logits and log-normalisers) must also give
    acceptance lengths in range."""
    cfg = QWEN3_8B_N2048
    gamma, T = 16, 1.0
    n = gamma - 1
    head = Head(cfg, gamma)
    h = head.inp.final_states(gamma)
    u, au, ru = head.inp.sample_uniforms(1, gamma)
    noise = head.inp.target_noise(1, gamma)
    d_g, z_g, l_g = head.sample(_dev(h), gamma, T, _dev(u))
    d_o, z_o, l_o, gap_o = O.sample_drafts(h, head.E64, T, u)
    check_drafts("chain drafts", cfg, T, d_g, z_g, l_g, d_o, z_o, l_o, gap_o)
    # the GPU's own chain
    t_g = torch.empty(cfg.B, gamma, cfg.V, dtype=torch.float32, device="cuda")
    noise_d = _dev(noise)
    t_g[:, :n] = z_g + 0.5 * noise_d[:, :n]
    t_g[:, n] = noise_d[:, n]
    tau_g, _ = accept_gpu(head.dims, cfg.B, gamma, T, d_g, z_g, t_g, _dev(au), _dev(ru), l_g)
    assert np.all((tau_g >= 1) & (tau_g <= gamma))
    # the verify on identical inputs
    z32 = np.ascontiguousarray(z_o, dtype=np.float32)
    t_o = build_target_logits_np(z32, noise)
    tau, nxt = accept_gpu(head.dims, cfg.B, gamma, T, _dev(d_o.astype(np.int32)), _dev(z32), _dev(t_o), _dev(au),
                          _dev(ru), None)
    check_accept("chain verify", tau, nxt, d_o, z32.astype(np.float64), t_o, T, au, ru)
    assert math.isfinite(float(tau.mean()))
