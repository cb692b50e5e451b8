"""GPU parity of the target side of a drafting iteration against the oracle:
dflash_target_verify (the target's causal verify pass over the anchor and the
drafts, with the hidden states of the tapped layers) and a closed speculative
loop in which the accepted tokens' tapped states become the drafter's new
context rows (fuse + inject) while the target keeps their K/V rows.

Both sides get the same seeded weights, context K/V and token inputs; the
tokens that drive a step (drafts, target tokens, acceptance lengths) are the
oracle's, so both sides follow one token stream and nothing the GPU computes
feeds the oracle.  Tolerances are those of tests/parity_util.py: stored tensors
(taps in the weight type, K/V rows in the cache type) with the stored-tensor
rule, target tokens wherever the oracle's top-2 gap is >= 1e-3, acceptance
lengths bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from block_diffusion_drafter_ctx_amd import binding as B
from block_diffusion_drafter_ctx_amd.runtime import DeviceDrafter, upload
from dflash_inputs import QWEN3_8B_N2048, Inputs, shrink
from oracle import dflash_oracle as O
from tests.parity_util import TOL, Workload, argmax_agree, close, close_rounded, close_stored, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU parity tests need a gfx950 GPU")
    B.load()


def target_cfg(**kw):
    """A target of 8 layers (taps 1..5), several weight tiles, GQA 4, ragged context."""
    base = dict(name="target_small", cid=401, D=512, L=8, Hq=8, Hkv=2, d=128, F=1536, V=1000, B=3,
                ctx=(37, 300, 1), gammas=(16,), gain_std=0.1)
    base.update(kw)
    return shrink(QWEN3_8B_N2048, **base)


class Target:
    """One synthetic target on both sides: weights, its own KV cache with a
    seeded random context, and the tapped layers."""

    def __init__(self, cfg, gamma_max, extra_rows=0):
        self.cfg = cfg
        self.inp = Inputs(cfg)
        self.dr = DeviceDrafter(cfg, self.inp, with_fusion=False)
        cap = (max(cfg.ctx) + gamma_max + extra_rows + 31) // 32 * 32
        self.cache = self.dr.cache(cfg.B, cap)
        self.dr.ensure_workspace(cfg.B, max(gamma_max, 2), 1)   # covers every verify of up to gamma_max rows
        f = lambda a: np.asarray(a, dtype=np.float64)  # noqa: E731
        self.o_layers = [dict(w_qkv=f(self.inp.w_qkv(l)), w_o=f(self.inp.w_o(l)), w_gateup=f(self.inp.w_gateup(l)),
                              w_down=f(self.inp.w_down(l)), g_attn=f(self.inp.g_attn(l)), g_ffn=f(self.inp.g_ffn(l)))
                         for l in range(cfg.L)]
        self.E = f(self.inp.embed())
        self.gf = f(self.inp.g_final())
        self.ocache = O.OracleCache(cfg.L, cfg.B, cfg.Hkv, cfg.d)
        rng = np.random.default_rng([cfg.cid, 5])
        for b, n in enumerate(cfg.ctx):
            k = O.store(rng.normal(0, 1, (cfg.L, n, cfg.Hkv, cfg.d)), cfg.cache_dtype)
            v = O.store(rng.normal(0, 1, (cfg.L, n, cfg.Hkv, cfg.d)), cfg.cache_dtype)
            if n:
                self.cache.put_rows(b, 0, k, v)
            for l in range(cfg.L):
                self.ocache.append(l, b, k[l], v[l])
        self.cache.set_lens(list(cfg.ctx))
        self.taps = O.tap_layers(cfg.L, cfg.n_tgt)

    def verify(self, tokens, tag):
        """Both sides' verify pass over tokens [B, gamma]; returns the oracle's result
        and the GPU's taps (device tensors)."""
        cfg = self.cfg
        Bn, g = tokens.shape
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        taps = [torch.full((Bn * g, cfg.D), float("nan"), dtype=dt, device="cuda") for _ in self.taps]
        tt = torch.full((Bn, g), -1, dtype=torch.int32, device="cuda")
        gap = torch.empty(Bn, g, dtype=torch.float32, device="cuda")
        lens = self.cache.len_list()
        before = [self.cache.snapshot(b, lens[b]) for b in range(Bn)]
        self.dr.target_verify(self.cache, torch.from_numpy(np.ascontiguousarray(tokens, dtype=np.int32)).cuda(), g,
                              self.taps, taps, tt, gap)
        torch.cuda.synchronize()
        assert self.cache.len_list() == lens
        for b in range(Bn):
            assert self.cache.same_rows(before[b], b, lens[b]), "target context rows changed"
        del before
        # the taps come back unrounded (and are rounded here, as the GPU stores them)
        res = O.target_verify(cfg, self.o_layers, self.gf, self.E, self.E, self.ocache, tokens, self.taps,
                              storage=cfg.cache_dtype, tap_storage="f64")
        excl = argmax_agree(tt.cpu().numpy(), res["tokens"], res["gap"], f"{tag} target tokens")
        assert np.abs(gap.cpu().numpy() - res["gap"]).max() <= TOL[cfg.dtype][0], f"{tag} top-2 gap"
        ties = 0
        for k, l in enumerate(self.taps):
            got = taps[k].float().cpu().numpy().reshape(Bn, g, cfg.D)
            ties += close_rounded(got, res["taps"][k], cfg.dtype, f"{tag} tap layer {l}")[2]
            res["taps"][k] = O.store(res["taps"][k], cfg.dtype)
        for b in range(Bn):
            gk, gv = self.cache.rows(b, lens[b], lens[b] + g)
            for l, (kb, vb) in enumerate(res["block_kv"]):
                close_stored(gk[l], kb[b], cfg.cache_dtype, f"{tag} target K l{l} b{b}", cfg.dtype)
                close_stored(gv[l], vb[b], cfg.cache_dtype, f"{tag} target V l{l} b{b}", cfg.dtype)
        log(f"{tag}: target tokens agree ({excl} near-tie rows excluded), taps {self.taps} match ({ties} near-tie "
            f"rounding flips beyond max-abs) and block K/V match")
        return res, taps, tt

    def commit(self, res, tau):
        """Keep the first tau[b] block rows of each sequence in the target cache."""
        lens = self.cache.len_list()
        for b, t in enumerate(tau):
            for l, (kb, vb) in enumerate(res["block_kv"]):
                self.ocache.append(l, b, kb[b][:t], vb[b][:t])
        self.cache.set_lens([n + int(t) for n, t in zip(lens, tau)])


def _tokens(cfg, gamma, seed):
    rng = np.random.default_rng([cfg.cid, 77, seed])
    return rng.integers(0, cfg.V, (cfg.B, gamma)).astype(np.int32)


def test_target_verify_small():
    cfg = target_cfg()
    log(f"target verify: {cfg.L} layers, taps {O.tap_layers(cfg.L)}, contexts {cfg.ctx}, gamma 16")
    t = Target(cfg, 16)
    t.verify(_tokens(cfg, 16, 0), "verify g16")


@pytest.mark.parametrize("gamma", [1, 2, 5, 33])
def test_target_verify_gamma_edges(gamma):
    # gamma 1 is a plain decoding step; 33 rows give 132 query rows per KV head
    cfg = target_cfg(cid=402, gammas=(gamma,))
    t = Target(cfg, gamma)
    t.verify(_tokens(cfg, gamma, 1), f"verify g{gamma}")


def test_target_verify_bf16_cache_head64_empty_context():
    cfg = target_cfg(cid=403, d=64, Hq=4, Hkv=4, ctx=(0, 70), B=2, V=777 * 2, cache_dtype="bf16")
    t = Target(cfg, 17)
    t.verify(_tokens(cfg, 17, 2), "verify bf16 cache d64 g17")
    cfg2 = target_cfg(cid=404, cache_dtype="bf16", ctx=(127, 128, 129))   # block rows across a key-range edge
    Target(cfg2, 16).verify(_tokens(cfg2, 16, 3), "verify bf16 cache g16")


def test_target_verify_f32_weights():
    cfg = target_cfg(cid=405, dtype="f32", D=256, Hq=4, Hkv=4, d=64, F=768, V=1024, ctx=(128, 9), B=2)
    Target(cfg, 16).verify(_tokens(cfg, 16, 4), "verify f32 g16")


@pytest.mark.timeout(900)
def test_target_verify_qwen3_8b_width():
    # the Qwen3-8B layer shape and vocabulary with 8 layers (taps 1..5), a
    # 2048-row context, one block of 16
    cfg = shrink(QWEN3_8B_N2048, name="target_qwen_width", cid=406, L=8, gain_std=0.1)
    log("target verify at the Qwen3-8B width: 8 layers, D 4096, V 151936, context 2048")
    Target(cfg, 16).verify(_tokens(cfg, 16, 5), "verify qwen width g16")


def greedy_continuation(tgt, anchors, n):
    """The target's own greedy continuation of each sequence, n tokens, by
    autoregressive decoding in the oracle (one row per verify, its K/V kept)."""
    cfg = tgt.cfg
    out = []
    for b, a in enumerate(anchors):
        c = tgt.ocache.prefix(b, tgt.ocache.lens()[b])
        seq = [int(a)]
        for _ in range(n):
            r = O.target_verify(cfg, tgt.o_layers, tgt.gf, tgt.E, tgt.E, c, np.array([[seq[-1]]]), [],
                                storage=cfg.cache_dtype)
            for l, (kb, vb) in enumerate(r["block_kv"]):
                c.append(l, 0, kb[0], vb[0])
            seq.append(int(r["tokens"][0, 0]))
        out.append(seq[1:])
    return np.array(out, dtype=np.int32)


def _speculative_loop(dcfg, tcfg, gamma, iters):
    """Drafter and target in a closed greedy loop on both sides: draft ->
    LM-head argmax -> target verify of (anchor, drafts) -> accept -> commit
    (the target keeps tau rows; the drafter fuses and injects the tau rows'
    tapped states).  The drafter shares the target's embedding and LM head.
    Random weights make the drafter and the target disagree (tau = 1), so on
    odd iterations the block carries the target's own greedy continuation
    instead of the drafts: every draft is then accepted (greedy speculative
    decoding is lossless) and whole blocks are committed."""
    tgt = Target(tcfg, gamma, extra_rows=iters * gamma)
    w = Workload(dcfg, gamma, iters, extra_cap=iters * gamma)
    # shared embedding / LM head: the target's
    w.dr.embed = tgt.dr.embed
    w.dr.weights.embed = w.dr.weights.lm_head = tgt.dr.embed.data_ptr()
    w.o_embed = tgt.E
    w.ingest(w.inp.ctx_states(), list(dcfg.ctx), "context")
    Bn, n = dcfg.B, gamma - 1
    anchors = w.inp.anchors() % tcfg.V
    taus = []
    for it in range(iters):
        # draft + argmax on both sides
        tokens = w.inp.block_tokens(gamma, anchors)
        h = torch.empty(Bn, gamma, dcfg.D, device="cuda")
        w.dr.draft(w.cache, torch.from_numpy(tokens).cuda(), None, gamma, h)
        d_g = torch.empty(Bn, n, dtype=torch.int32, device="cuda")
        w.dr.argmax_accept(B.ARGMAX, h, Bn, gamma, d_g)
        torch.cuda.synchronize()
        hf_o, _ = O.draft_forward(dcfg, w.o_layers, w.o_gfinal, w.ocache, gamma, embed=w.o_embed, tokens=tokens,
                                  storage=dcfg.cache_dtype)
        d_o, gap_o, _ = O.lm_head_argmax(hf_o, w.o_embed)
        close(h.cpu().numpy(), hf_o, dcfg.dtype, f"loop it{it} drafter h_final")
        argmax_agree(d_g.cpu().numpy(), d_o, gap_o, f"loop it{it} drafts")
        if it % 2 == 1:
            d_o = greedy_continuation(tgt, anchors, n)
        # the target verifies the oracle's block on both sides
        block = np.concatenate([anchors[:, None], d_o], axis=1).astype(np.int32)
        res, taps, _ = tgt.verify(block, f"loop it{it}")
        # greedy acceptance on identical tokens
        tau = torch.empty(Bn, dtype=torch.int32, device="cuda")
        nxt = torch.empty(Bn, dtype=torch.int32, device="cuda")
        w.dr.argmax_accept(B.ACCEPT, None, Bn, gamma, torch.from_numpy(np.ascontiguousarray(d_o)).cuda(),
                           target=torch.from_numpy(np.ascontiguousarray(res["tokens"])).cuda(), tau=tau, nxt=nxt)
        torch.cuda.synchronize()
        tau_o, nxt_o = O.accept(d_o, res["tokens"])
        assert np.array_equal(tau.cpu().numpy(), tau_o) and np.array_equal(nxt.cpu().numpy(), nxt_o)
        if it % 2 == 1:
            assert np.all(tau_o == gamma), f"the target's own continuation must be accepted whole: {tau_o}"
        # commit: the target keeps tau rows; the drafter appends their tapped states
        tgt.commit(res, tau_o)
        rows = [slice(b * gamma, b * gamma + int(tau_o[b])) for b in range(Bn)]
        h_dev = [torch.cat([t[r] for r in rows]).contiguous() for t in taps]
        h_ora = [np.concatenate([res["taps"][k][b][:int(tau_o[b])] for b in range(Bn)]) for k in range(len(taps))]
        append_context(w, h_dev, h_ora, [int(x) for x in tau_o], f"loop it{it} append")
        taus.append(tau_o.tolist())
        anchors = nxt_o
    log(f"speculative loop: tau per iteration {taus}")
    return taus


def append_context(w, h_dev, h_ora, counts, tag):
    """Fuse + inject appended target states on both sides, each side its own
    states (device tensors on the GPU, the oracle's arrays in the oracle)."""
    cfg = w.cfg
    T = sum(counts)
    H_t = w.dr.context_buffer(T)
    lens_before = w.cache.len_list()
    w.dr.ensure_workspace(cfg.B, w.gamma, max(cfg.n_ctx_total, T, 1))
    w.dr.fuse(h_dev, T, H_t)
    w.dr.inject(H_t, counts, w.cache)
    torch.cuda.synchronize()
    Ht_o = O.fuse_context(h_ora, w.o_wc, w.o_gc, cfg.eps, w.st)
    close_stored(H_t.float().cpu().numpy(), Ht_o, w.st, f"{tag} H_t", w.tol)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(int)
    for b in range(cfg.B):
        gk, gv = w.cache.rows(b, lens_before[b], lens_before[b] + counts[b])
        for l in range(cfg.L):
            k, v = O.inject_kv(Ht_o[off[b]:off[b + 1]], w.o_layers[l]["w_qkv"], cfg.Hq, cfg.Hkv, cfg.d, w.st)
            w.ocache.append(l, b, k, v)
            close_stored(gk[l], k, w.st, f"{tag} K l{l} b{b}", w.tol)
            close_stored(gv[l], v, w.st, f"{tag} V l{l} b{b}", w.tol)
    assert w.cache.len_list() == [a + c for a, c in zip(lens_before, counts)]


def test_speculative_loop_small():
    tcfg = target_cfg(cid=410, B=2, ctx=(40, 97))
    dcfg = shrink(QWEN3_8B_N2048, name="drafter_small", cid=411, D=512, L=2, Hq=8, Hkv=2, d=128, F=1536, V=1000,
                  B=2, ctx=(40, 97), gammas=(8,), gain_std=0.1)
    taus = _speculative_loop(dcfg, tcfg, 8, 4)
    assert all(1 <= t <= 8 for row in taus for t in row)
    assert taus[1] == [8, 8] and taus[3] == [8, 8]


def test_speculative_loop_bf16_cache():
    tcfg = target_cfg(cid=412, B=2, ctx=(33, 64), cache_dtype="bf16")
    dcfg = shrink(QWEN3_8B_N2048, name="drafter_small_bf16", cid=413, D=512, L=2, Hq=8, Hkv=2, d=128, F=1536,
                  V=1000, B=2, ctx=(33, 64), gammas=(16,), gain_std=0.1, cache_dtype="bf16")
    _speculative_loop(dcfg, tcfg, 16, 4)
