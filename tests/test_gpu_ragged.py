"""Blocks with a length per sequence: the HIP path against the CPU oracle.

Same tolerances as the uniform parity tests (tests/parity_util.py): per
compared tensor max-abs 2e-2 and relative 1e-2 for bf16 workloads (1e-4 /
1e-5 for fp32), stored tensors within one storage ulp on at most 0.1% of
elements, drafts equal wherever the oracle's top-2 gap is at least 1e-3 (3e-2
with a bf16 cache), acceptance bit-exact on identical token inputs.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from block_diffusion_drafter_ctx_amd import binding as B
from dflash_inputs import BATCH16_RAGGED, DEEP8_B4_N8192, LONG_CTX_N32768, QWEN3_8B_N2048, TINY_F32, shrink
from oracle import dflash_oracle as O
from tests.parity_util import (TOL, Workload, argmax_agree, close, close_stored,
                               log)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU parity tests need a gfx950 GPU")
    B.load()


def small(**kw):
    base = dict(name="small_bf16_ragged", cid=120, D=512, L=2, Hq=8, Hkv=2, d=128, F=1536, V=1000, B=4,
                ctx=(37, 300, 1, 64), gammas=(16,), gain_std=0.1, iters=1)
    base.update(kw)
    return shrink(QWEN3_8B_N2048, **base)


class Ragged(Workload):
    """A seeded workload whose sequences draft blocks of their own lengths."""

    def __init__(self, cfg, gammas, override=False):
        assert len(gammas) == cfg.B
        super().__init__(cfg, max(gammas), 1, override=override)
        self.gammas = [int(g) for g in gammas]

    def ragged_iteration(self, tag="ragged"):
        cfg, gs, dev = self.cfg, self.gammas, self.dev
        Bn, D, V = cfg.B, cfg.D, cfg.V
        off = np.concatenate([[0], np.cumsum(gs)]).astype(int)
        M = int(off[-1])
        anchors = self.inp.anchors()
        toks = [np.array([anchors[b]] + [cfg.mask_id] * (g - 1), dtype=np.int32) for b, g in enumerate(gs)]
        tok_dev = torch.from_numpy(np.concatenate(toks)).to(dev)
        ovs = ov_dev = None
        if self.override:
            full = self.inp.embed_override(max(gs))
            ovs = [np.ascontiguousarray(full[b, :g]) for b, g in enumerate(gs)]
            ov_dev = torch.from_numpy(np.concatenate(ovs)).to(dev)
        h_final = torch.empty(M, D, dtype=torch.float32, device=dev)
        lens = self.cache.len_list()
        before = [self.cache.snapshot(b, lens[b]) for b in range(Bn)]
        self.dr.draft_ragged(self.cache, tok_dev, ov_dev, gs, h_final)
        nd = M - Bn
        draft = torch.empty(nd, dtype=torch.int32, device=dev)
        logits = torch.empty(nd, V, dtype=torch.float32, device=dev)
        gap = torch.empty(nd, dtype=torch.float32, device=dev)
        self.dr.argmax_accept_ragged(B.ARGMAX, h_final, gs, draft, logits=logits, gap=gap)
        draft_lean = torch.empty_like(draft)
        self.dr.argmax_accept_ragged(B.ARGMAX, h_final, gs, draft_lean)
        torch.cuda.synchronize()
        assert torch.equal(draft, draft_lean), "argmax differs when logits / gap are not requested"
        assert self.cache.len_list() == lens
        for b in range(Bn):
            assert self.cache.same_rows(before[b], b, lens[b]), "context K/V rows changed"
        del before
        # oracle: each sequence's one-sequence pass over its own block
        hf_o, kv_o = O.draft_forward_ragged(cfg, self.o_layers, self.o_gfinal, self.ocache, gs, embed=self.o_embed,
                                            tokens=toks, override=ovs, storage=self.st)
        d_o, gap_o, z_o = O.lm_head_argmax_ragged(hf_o, self.o_embed)
        hg = h_final.cpu().numpy()
        e = close(hg, np.concatenate(hf_o), self.tol, f"{tag} h_final")
        close(logits.cpu().numpy(), np.concatenate(z_o), self.tol, f"{tag} logits")
        for b in range(Bn):
            gk, gv = self.cache.rows(b, lens[b], lens[b] + gs[b])
            for l in range(cfg.L):
                close_stored(gk[l], kv_o[b][l][0], self.st, f"{tag} block K l{l} b{b}", self.tol)
                close_stored(gv[l], kv_o[b][l][1], self.st, f"{tag} block V l{l} b{b}", self.tol)
        dcat, gcat = np.concatenate(d_o), np.concatenate(gap_o)
        excl = argmax_agree(draft.cpu().numpy(), dcat, gcat, f"{tag} drafts")
        assert np.abs(gap.cpu().numpy() - gcat).max() <= TOL[self.tol][0]
        # acceptance on the oracle's drafts and synthetic targets built from them
        rng = np.random.default_rng([cfg.cid, 77])
        targets = []
        for b, g in enumerate(gs):
            n = g - 1
            match = rng.random(n) < 0.8
            t = np.where(match, d_o[b], (d_o[b] + rng.integers(1, V, n)) % V)
            targets.append(np.concatenate([t, [rng.integers(0, V)]]).astype(np.int32))
        tgt_dev = torch.from_numpy(np.concatenate(targets)).to(dev)
        d_dev = torch.from_numpy(dcat.astype(np.int32)).to(dev)
        tau = torch.full((Bn,), -1, dtype=torch.int32, device=dev)
        nxt = torch.full((Bn,), -1, dtype=torch.int32, device=dev)
        self.dr.argmax_accept_ragged(B.ACCEPT, None, gs, d_dev, target=tgt_dev, tau=tau, nxt=nxt)
        torch.cuda.synchronize()
        tau_o, nxt_o = O.accept_ragged(d_o, targets)
        assert np.array_equal(tau.cpu().numpy(), tau_o) and np.array_equal(nxt.cpu().numpy(), nxt_o)
        assert np.all((tau_o >= 1) & (tau_o <= np.array(gs)))
        log(f"{tag}: gammas {gs}: h_final err {e[0]:.2e}, drafts agree ({excl} near-tie rows excluded), "
            f"tau {tau_o.tolist()}")
        return h_final, draft, logits

    def run_ragged(self):
        self.ingest(self.inp.ctx_states(), list(self.cfg.ctx), "context")
        return self.ragged_iteration()


def test_ragged_small_tokens():
    # block lengths 2 (one draft), 16, 5 and 33 (two row groups of queries)
    log("ragged small bf16, token embeddings")
    Ragged(small(), [2, 16, 5, 33]).run_ragged()


def test_ragged_small_override_bf16_cache():
    log("ragged small bf16, override rows, bf16 cache")
    Ragged(small(cid=121, B=3, ctx=(100, 0, 17), cache_dtype="bf16"), [7, 3, 17], override=True).run_ragged()


def test_ragged_head64():
    log("ragged small bf16, head_dim 64, GQA 1")
    Ragged(small(cid=122, d=64, Hq=4, Hkv=4, B=3, ctx=(0, 70, 5), V=777 * 2), [9, 2, 4], override=True).run_ragged()


def test_ragged_f32():
    log("ragged tiny fp32 drafter")
    cfg = shrink(TINY_F32, cid=123, B=3, ctx=(128, 40, 0), gain_std=0.1)
    Ragged(cfg, [16, 4, 9], override=True).run_ragged()


def test_ragged_register_k():
    # 13 block rows (register-K gate/up) and 11 LM-head rows (register-K head
    # with the top-2 epilogue) over two sequences
    log("ragged register-K shapes: D=2048, 2F=16384, V=20001")
    cfg = small(cid=124, D=2048, L=1, Hq=16, Hkv=4, F=8192, V=20001, B=2, ctx=(256, 31))
    Ragged(cfg, [5, 8], override=True).run_ragged()


def test_ragged_equal_lengths_match_uniform_bit_for_bit():
    cfg = small(cid=125, B=3, ctx=(37, 300, 1))
    w = Ragged(cfg, [16, 16, 16], override=True)
    w.ingest(w.inp.ctx_states(), list(cfg.ctx), "context")
    h_r, d_r, z_r = w.ragged_iteration("ragged-as-uniform")
    ov = torch.from_numpy(w.inp.embed_override(16)).to("cuda")
    h_u = torch.empty(cfg.B, 16, cfg.D, dtype=torch.float32, device="cuda")
    w.dr.draft(w.cache, None, ov, 16, h_u)
    d_u = torch.empty(cfg.B, 15, dtype=torch.int32, device="cuda")
    z_u = torch.empty(cfg.B, 15, cfg.V, dtype=torch.float32, device="cuda")
    w.dr.argmax_accept(B.ARGMAX, h_u, cfg.B, 16, d_u, logits=z_u)
    torch.cuda.synchronize()
    assert torch.equal(h_r, h_u.reshape(-1, cfg.D))
    assert torch.equal(d_r, d_u.reshape(-1)) and torch.equal(z_r, z_u.reshape(-1, cfg.V))


def test_ragged_full_batch16():
    # the batch16_ragged workload (16 sequences, contexts U[1024, 4096]) at the
    # full Qwen3-8B shape, with block lengths 4, 8, 16, 32 cycling over it
    cfg = BATCH16_RAGGED
    gammas = [4, 8, 16, 32] * 4
    log(f"ragged full batch16: gammas {gammas}")
    Ragged(cfg, gammas).run_ragged()


def test_ragged_max_batch():
    # 64 sequences (the most one call takes) with block lengths drawn over the
    # whole allowed range [2, 33] and contexts from empty to 200 rows
    rng = np.random.default_rng(126)
    ctx = tuple(int(c) for c in rng.integers(0, 201, 64))
    gammas = [int(g) for g in rng.integers(2, 34, 64)]
    log(f"ragged 64 sequences: gammas {gammas[:8]}..., contexts {ctx[:8]}...")
    Ragged(small(cid=126, B=64, ctx=ctx), gammas).run_ragged()
