"""Shared driver for the GPU-vs-oracle parity tests.

``Workload`` runs the same seeded workload through the HIP path (via the C ABI)
and through the CPU oracle, stage by stage, and records every comparison.
Tolerances (per compared tensor, both must hold):
  bf16 storage: max |gpu - oracle| <= 2e-2 and ||gpu - oracle|| / ||oracle|| <= 1e-2
  fp32 storage: max-abs <= 1e-4 and relative <= 1e-5
Tensors *stored* in bf16 (H_t, cache K/V, block K/V) are compared the same way,
except that an element may also differ by exactly one bf16 ulp of the oracle's
value (both sides rounded nearly equal values to neighbouring bf16 numbers; at
|x| >= 4 one ulp is 0.031 > 2e-2), and at most 0.1% of elements may do so
(tests/test_storage_rounding_pin.py measures this between two correct
evaluations at the Qwen3-8B shape).
Argmax ids must agree on every row whose oracle top-2 gap is >= 1e-3, for an
fp32 and a bf16 cache alike (the same pin shows two correct bf16-cache
evaluations ~2e-3 apart in the logits at most, with no argmax disagreement
above that gap); acceptance lengths and next anchors must match bit for bit
given the same draft and target tokens.
"""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

from block_diffusion_drafter_ctx_amd import binding as B
from block_diffusion_drafter_ctx_amd.runtime import DeviceDrafter, upload
from dflash_inputs import Inputs, build_target_np
from oracle import dflash_oracle as O

TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-5)}
GAP_MIN = 1e-3


def log(msg):
    print(f"[parity {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def close(got, ref, dtype, what):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    mx, rl = TOL[dtype]
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / den) if den > 0 else err
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert err <= mx and rel <= rl, f"{what}: max-abs {err:.3e} (tol {mx}), rel {rel:.3e} (tol {rl})"
    return err, rel


def bf16_ulp(x):
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 7)


def close_stored(got, ref, dtype, what, tol=None):
    """close() for tensors held in the storage type ``dtype`` (one-ulp rounding
    flips allowed for bf16); ``tol`` is the tolerance class (default ``dtype``)."""
    tol = dtype if tol is None else tol
    if dtype != "bf16":
        return close(got, ref, tol, what)
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    mx, rl = TOL[tol]
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    diff = np.abs(got - ref)
    over = diff > mx
    flips = over & (diff <= bf16_ulp(ref) * (1 + 1e-9))
    bad = over & ~flips
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / den) if den > 0 else float(diff.max(initial=0.0))
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond max-abs {mx} and one bf16 ulp " \
                          f"(worst {float(diff[bad].max()):.3e})"
    frac = float(flips.mean()) if flips.size else 0.0
    assert frac <= 1e-3, f"{what}: {frac:.2e} of elements are one-ulp flips (limit 1e-3)"
    assert rel <= rl, f"{what}: rel {rel:.3e} (tol {rl})"
    return float(diff.max(initial=0.0)), rel


def close_rounded(got, exact, dtype, what, tol=None, eps=1e-4):
    """A tensor stored in ``dtype`` against the oracle's unrounded values.  The
    tolerance class ``tol`` applies to the oracle's stored value r = store(x);
    beyond it an element may only be r's neighbour in the storage type on the
    other side of x, when x lies within eps * |x| of the midpoint between the
    two (a rounding decision the two sides' accumulation errors may take
    either way).  No share of such elements is capped: each must be a near-tie."""
    tol = dtype if tol is None else tol
    x = np.asarray(exact, dtype=np.float64)
    r = O.store(x, dtype)
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == x.shape, (what, got.shape, x.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    mx, rl = TOL[tol]
    diff = np.abs(got - r)
    over = diff > mx
    if over.any():
        g, rr, xx = got[over], r[over], x[over]
        ulp = bf16_ulp(np.minimum(np.abs(g), np.abs(rr))) if dtype == "bf16" else np.spacing(np.abs(rr).astype(np.float32)).astype(np.float64)
        neighbour = np.abs(g - rr) <= ulp * (1 + 1e-9)
        bracket = (np.minimum(g, rr) <= xx) & (xx <= np.maximum(g, rr))
        near_tie = np.abs(xx - 0.5 * (g + rr)) <= eps * np.abs(xx)
        bad = ~(neighbour & bracket & near_tie)
        assert not bad.any(), (f"{what}: {int(bad.sum())} of {int(over.sum())} elements beyond max-abs {mx} are not "
                               f"near-tie neighbours (worst |x - midpoint| / |x| "
                               f"{float(np.max(np.abs(xx - 0.5 * (g + rr))[bad] / np.abs(xx[bad]))):.2e})")
    den = float(np.linalg.norm(r))
    rel = float(np.linalg.norm(got - r) / den) if den > 0 else float(diff.max(initial=0.0))
    assert rel <= rl, f"{what}: rel {rel:.3e} (tol {rl})"
    return float(diff.max(initial=0.0)), rel, int(over.sum())


def argmax_agree(gpu_ids, ora_ids, ora_gap, what, gap_min=GAP_MIN):
    gpu_ids = np.asarray(gpu_ids).reshape(-1)
    ora_ids = np.asarray(ora_ids).reshape(-1)
    gap = np.asarray(ora_gap).reshape(-1)
    sure = gap >= gap_min
    bad = np.nonzero(sure & (gpu_ids != ora_ids))[0]
    assert bad.size == 0, f"{what}: argmax differs on rows {bad[:10]} (gaps {gap[bad[:10]]})"
    return int((~sure).sum())


class Workload:
    """One seeded workload on both sides.  ``cfg`` is a dflash_inputs.Config."""

    def __init__(self, cfg, gamma, iters, device="cuda", override=False, extra_cap=0):
        self.cfg, self.gamma, self.iters, self.override = cfg, gamma, iters, override
        self.tol = cfg.dtype            # tolerance class: the weight / compute type
        self.st = cfg.cache_dtype       # storage rounding of H_t and the cache
        self.inp = Inputs(cfg)
        self.dev = device
        t0 = time.time()
        self.dr = DeviceDrafter(cfg, self.inp, device)
        cap = max(cfg.ctx) + iters * cfg.append_rows + max(gamma, cfg.append_rows) + extra_cap
        cap = (cap + 31) // 32 * 32
        self.cache = self.dr.cache(cfg.B, cap)
        self.dr.ensure_workspace(cfg.B, gamma, max(cfg.n_ctx_total, cfg.B * cfg.append_rows, 1))
        # oracle weights in float64 (converted once)
        f = lambda a: np.asarray(a, dtype=np.float64)  # noqa: E731
        self.o_layers = [dict(w_qkv=f(self.inp.w_qkv(l)), w_o=f(self.inp.w_o(l)), w_gateup=f(self.inp.w_gateup(l)),
                              w_down=f(self.inp.w_down(l)), g_attn=f(self.inp.g_attn(l)), g_ffn=f(self.inp.g_ffn(l)))
                         for l in range(cfg.L)]
        self.o_embed = f(self.inp.embed())
        self.o_gfinal = f(self.inp.g_final())
        self.o_wc = self.inp.w_c()
        self.o_gc = self.inp.g_c()
        self.ocache = O.OracleCache(cfg.L, cfg.B, cfg.Hkv, cfg.d)
        self.report = {}
        log(f"{cfg.name}: setup {time.time() - t0:.1f}s (cap {cap})")

    # ------------------------------------------------------------- context
    def seq_rows(self, counts):
        off = np.concatenate([[0], np.cumsum(counts)]).astype(int)
        return [(int(off[b]), int(off[b + 1])) for b in range(len(counts))]

    def ingest(self, states, counts, tag):
        """Fuse + inject ``states`` (n_tgt arrays [sum(counts), D]) on both sides."""
        cfg = self.cfg
        T = int(sum(counts))
        if T == 0:
            return
        h_dev = [upload(h, cfg, self.dev) for h in states]
        H_t = self.dr.context_buffer(T)
        lens_before = self.cache.len_list()
        self.dr.fuse(h_dev, T, H_t)
        self.dr.inject(H_t, counts, self.cache)
        torch.cuda.synchronize()
        assert self.cache.len_list() == [a + c for a, c in zip(lens_before, counts)]
        Ht_o = O.fuse_context(states, self.o_wc, self.o_gc, cfg.eps, self.st)
        self.report[f"{tag}/H_t"] = close_stored(H_t.float().cpu().numpy(), Ht_o, self.st, f"{tag} H_t", self.tol)
        for b, (lo, hi) in enumerate(self.seq_rows(counts)):
            n0 = lens_before[b]
            gk, gv = self.cache.rows(b, n0, n0 + hi - lo)
            for l in range(cfg.L):
                k, v = O.inject_kv(Ht_o[lo:hi], self.o_layers[l]["w_qkv"], cfg.Hq, cfg.Hkv, cfg.d, self.st)
                self.ocache.append(l, b, k, v)
                if hi > lo:
                    close_stored(gk[l], k, self.st, f"{tag} K l{l} b{b}", self.tol)
                    close_stored(gv[l], v, self.st, f"{tag} V l{l} b{b}", self.tol)
        assert self.cache.len_dev.cpu().tolist() == self.cache.len_list(), "device length mirror"
        log(f"{tag}: {T} rows fused + injected, cache matches")

    # ------------------------------------------------------------- drafting
    def draft_iteration(self, it, anchors):
        cfg, g = self.cfg, self.gamma
        Bn, n = cfg.B, g - 1
        tokens = self.inp.block_tokens(g, anchors)
        tok_dev = torch.from_numpy(tokens).to(self.dev)
        ov = self.inp.embed_override(g) if self.override else None
        ov_dev = torch.from_numpy(ov).to(self.dev) if ov is not None else None
        h_final = torch.empty(Bn, g, cfg.D, dtype=torch.float32, device=self.dev)
        lens = self.cache.len_list()
        before = [self.cache.snapshot(b, lens[b]) for b in range(Bn)]
        self.dr.draft(self.cache, tok_dev, ov_dev, g, h_final)
        draft = torch.empty(Bn, n, dtype=torch.int32, device=self.dev)
        logits = torch.empty(Bn, n, cfg.V, dtype=torch.float32, device=self.dev)
        gap = torch.empty(Bn, n, dtype=torch.float32, device=self.dev)
        self.dr.argmax_accept(B.ARGMAX, h_final, Bn, g, draft, logits=logits, gap=gap)
        # the same argmax without the debug outputs (the path a drafting loop takes)
        draft_lean = torch.empty_like(draft)
        self.dr.argmax_accept(B.ARGMAX, h_final, Bn, g, draft_lean)
        torch.cuda.synchronize()
        assert torch.equal(draft, draft_lean), "argmax differs when logits / gap are not requested"
        assert self.cache.len_list() == lens
        for b in range(Bn):
            assert self.cache.same_rows(before[b], b, lens[b]), "context K/V rows changed"
        del before
        # oracle
        hf_o, block_kv = O.draft_forward(cfg, self.o_layers, self.o_gfinal, self.ocache, g, embed=self.o_embed,
                                         tokens=tokens, override=ov, storage=self.st)
        d_o, gap_o, logits_o = O.lm_head_argmax(hf_o, self.o_embed)
        tag = f"it{it}"
        hg = h_final.cpu().numpy()
        lg = logits.cpu().numpy()
        gg = gap.cpu().numpy()
        d_g = draft.cpu().numpy()
        e_h = np.abs(hg - hf_o)
        e_l = np.abs(lg - logits_o)
        log(f"{tag}: h_final max-abs {e_h.max():.3e} rel {np.linalg.norm(hg - hf_o) / np.linalg.norm(hf_o):.3e}; "
            f"logits max-abs {e_l.max():.3e} mean-abs {e_l.mean():.3e}; gap max-abs {np.abs(gg - gap_o).max():.3e}; "
            f"oracle gaps min {gap_o.min():.3e}")
        self.report[f"{tag}/h_final"] = close(hg, hf_o, self.tol, f"{tag} h_final")
        self.report[f"{tag}/logits_maxabs"] = float(e_l.max())
        close(lg, logits_o, self.tol, f"{tag} logits")
        # every layer's block K/V rows stay in that layer's cache scratch rows
        for b in range(Bn):
            gk, gv = self.cache.rows(b, lens[b], lens[b] + g)
            for l, (kb_o, vb_o) in enumerate(block_kv):
                close_stored(gk[l], kb_o[b], self.st, f"{tag} block K l{l} b{b}", self.tol)
                close_stored(gv[l], vb_o[b], self.st, f"{tag} block V l{l} b{b}", self.tol)
        excl = argmax_agree(d_g, d_o, gap_o, f"{tag} drafts")
        # the gap is a difference of two logits: compared in absolute terms only
        gmx = TOL[self.tol][0]
        assert np.abs(gg - gap_o).max() <= gmx, f"{tag} top2 gap: max-abs {np.abs(gg - gap_o).max():.3e}"
        # accept on identical token inputs on both sides: the oracle's drafts and
        # the synthetic targets built from them (nothing of the GPU's feeds the oracle)
        match, r, bonus = self.inp.verify_draws(it, g)
        target = build_target_np(d_o, match, r, bonus, cfg.V)
        tgt_dev = torch.from_numpy(target).to(self.dev)
        d_o_dev = torch.from_numpy(np.ascontiguousarray(d_o, dtype=np.int32)).to(self.dev)
        tau = torch.empty(Bn, dtype=torch.int32, device=self.dev)
        nxt = torch.empty(Bn, dtype=torch.int32, device=self.dev)
        self.dr.argmax_accept(B.ACCEPT, None, Bn, g, d_o_dev, target=tgt_dev, tau=tau, nxt=nxt)
        torch.cuda.synchronize()
        tau_o, nxt_o = O.accept(d_o, target)
        assert np.array_equal(tau.cpu().numpy(), tau_o), (tau.cpu().numpy(), tau_o)
        assert np.array_equal(nxt.cpu().numpy(), nxt_o)
        assert np.all((tau_o >= 1) & (tau_o <= n + 1))
        log(f"{tag}: h_final err {self.report[f'{tag}/h_final'][0]:.2e}, drafts agree "
            f"({excl} near-tie rows excluded), tau {tau_o.tolist()}")
        return nxt_o, h_final, draft

    def run_gammas(self, gammas):
        """Ingest the context once, then one drafting pass per block length on it
        (no appends: every pass sees the same cache)."""
        self.ingest(self.inp.ctx_states(), list(self.cfg.ctx), "context")
        anchors = self.inp.anchors()
        for g in gammas:
            self.gamma = g
            self.draft_iteration(0, anchors)
        return self.report

    def run(self, iters=None):
        cfg = self.cfg
        self.ingest(self.inp.ctx_states(), list(cfg.ctx), "context")
        anchors = self.inp.anchors()
        for it in range(self.iters if iters is None else iters):
            anchors, _, _ = self.draft_iteration(it, anchors)
            if cfg.append_rows:
                self.ingest(self.inp.append_states(it), [cfg.append_rows] * cfg.B, f"append{it}")
        return self.report
