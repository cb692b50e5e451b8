"""Many anchored blocks at once (the training-style mask): HIP path against
the CPU oracle.  Tolerances as in tests/parity_util.py."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

from block_diffusion_drafter_ctx_amd import binding as B
from dflash_inputs import BATCH16_RAGGED, DEEP8_B4_N8192, LONG_CTX_N32768, QWEN3_8B_N2048, TINY_F32, shrink
from oracle import dflash_oracle as O
from tests.parity_util import Workload, argmax_agree, close, close_stored, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU parity tests need a gfx950 GPU")
    B.load()


def small(**kw):
    base = dict(name="small_bf16_blocks", cid=130, D=512, L=2, Hq=8, Hkv=2, d=128, F=1536, V=1000, B=2,
                ctx=(37, 300), gammas=(16,), gain_std=0.1, iters=1, append_rows=0)
    base.update(kw)
    return shrink(QWEN3_8B_N2048, **base)


def block_rows(blocks, lens, g, pairs):
    """(sequence, first scratch row) of each block, by the documented layout:
    slots from each sequence's context length rounded up to 32, in call order;
    with pairs, two consecutive blocks of one sequence share a slot of 2g rows
    rounded up to 32, the second block's rows right after the first's."""
    nxt = {s: (n + 31) // 32 * 32 for s, n in enumerate(lens)}
    out, k = [], 0
    while k < len(blocks):
        s = blocks[k][0]
        two = pairs and k + 1 < len(blocks) and blocks[k + 1][0] == s
        pos = nxt[s]
        nxt[s] += ((2 * g if two else g) + 31) // 32 * 32
        out.append((s, pos))
        if two:
            out.append((s, pos + g))
        k += 2 if two else 1
    return out


class Blocks(Workload):
    """A seeded context, then blocks anchored inside it."""

    def __init__(self, cfg, blocks, gamma, override=False):
        g32 = (gamma + 31) // 32 * 32
        per_seq = max(sum(1 for s, _ in blocks if s == b) for b in range(cfg.B))
        super().__init__(cfg, gamma, 1, override=override, extra_cap=32 + per_seq * g32)
        self.blocks = [(int(s), int(a)) for s, a in blocks]
        # two consecutive blocks of a sequence share a query group with bf16 weights and an fp32 cache
        self.pairs = (cfg.dtype == "bf16" and cfg.cache_dtype == "f32" and 2 * (cfg.Hq // cfg.Hkv) * gamma <= 128
                      and os.environ.get("DFLASH_BLOCK_PAIRS") != "2")
        self.dr.ensure_workspace(max(cfg.B, len(blocks)), gamma, max(cfg.n_ctx_total, 1))

    def run_blocks(self, tag="blocks"):
        cfg, g, dev = self.cfg, self.gamma, self.dev
        self.ingest(self.inp.ctx_states(), list(cfg.ctx), "context")
        nb = len(self.blocks)
        rng = np.random.default_rng([cfg.cid, 91])
        toks = np.full((nb, g), cfg.mask_id, dtype=np.int32)
        toks[:, 0] = rng.integers(0, cfg.V - 1, nb)
        ov = rng.normal(0, 1, (nb, g, cfg.D)).astype(np.float32) if self.override else None
        h_final = torch.empty(nb, g, cfg.D, dtype=torch.float32, device=dev)
        lens = self.cache.len_list()
        before = [self.cache.snapshot(b, lens[b]) for b in range(cfg.B)]
        seqs = [s for s, _ in self.blocks]
        anchors = [a for _, a in self.blocks]
        self.dr.draft_blocks(self.cache, seqs, anchors, g, torch.from_numpy(toks).to(dev),
                             None if ov is None else torch.from_numpy(ov).to(dev), h_final)
        draft = torch.empty(nb, g - 1, dtype=torch.int32, device=dev)
        logits = torch.empty(nb, g - 1, cfg.V, dtype=torch.float32, device=dev)
        gap = torch.empty(nb, g - 1, dtype=torch.float32, device=dev)
        self.dr.argmax_accept(B.ARGMAX, h_final, nb, g, draft, logits=logits, gap=gap)
        torch.cuda.synchronize()
        assert self.cache.len_list() == lens
        for b in range(cfg.B):
            assert self.cache.same_rows(before[b], b, lens[b]), "context K/V rows changed"
        del before
        hf_o, kv_o = O.draft_forward_blocks(cfg, self.o_layers, self.o_gfinal, self.ocache, self.blocks, g,
                                            embed=self.o_embed, tokens=toks, override=ov, storage=self.st)
        e = close(h_final.cpu().numpy(), hf_o, self.tol, f"{tag} h_final")
        d_o, gap_o, z_o = O.lm_head_argmax(hf_o, self.o_embed)
        close(logits.cpu().numpy(), z_o, self.tol, f"{tag} logits")
        excl = argmax_agree(draft.cpu().numpy(), d_o, gap_o, f"{tag} drafts")
        # each block's own K/V rows sit in its scratch slot past its sequence's context
        for k, (s, pos) in enumerate(block_rows(self.blocks, lens, g, self.pairs)):
            gk, gv = self.cache.rows(s, pos, pos + g)
            for l in range(cfg.L):
                close_stored(gk[l], kv_o[k][l][0], self.st, f"{tag} block {k} K l{l}", self.tol)
                close_stored(gv[l], kv_o[k][l][1], self.st, f"{tag} block {k} V l{l}", self.tol)
        log(f"{tag}: {nb} blocks {self.blocks[:8]}: h_final err {e[0]:.2e}, drafts agree "
            f"({excl} near-tie rows excluded)")


def test_blocks_small():
    # anchors at 0 (no context), inside, and at the full length; three blocks
    # per sequence share its scratch region
    blocks = [(0, 0), (0, 20), (1, 150), (1, 300), (0, 37), (1, 1)]
    log("anchored blocks, small bf16")
    Blocks(small(), blocks, 16).run_blocks()


def test_blocks_override_bf16_cache_gamma33():
    blocks = [(0, 12), (1, 299), (1, 64), (0, 36)]
    log("anchored blocks, bf16 cache, gamma 33 (two row groups)")
    Blocks(small(cid=131, cache_dtype="bf16"), blocks, 33, override=True).run_blocks()


def test_blocks_unpaired_gamma20():
    # 2 * G * gamma = 160 query rows would not fit one attention workgroup:
    # consecutive blocks stay one to a group (fp32 cache)
    blocks = [(0, 30), (0, 7), (1, 200), (1, 250), (0, 37)]
    log("anchored blocks, gamma 20 (no pairs)")
    Blocks(small(cid=136), blocks, 20).run_blocks()


def test_blocks_head64():
    blocks = [(0, 5), (0, 0), (1, 70)]
    log("anchored blocks, head_dim 64")
    Blocks(small(cid=132, d=64, Hq=4, Hkv=4, ctx=(9, 70)), blocks, 8, override=True).run_blocks()


def test_blocks_f32():
    blocks = [(0, 100), (0, 3), (0, 128)]
    log("anchored blocks, tiny fp32 drafter")
    cfg = shrink(TINY_F32, cid=133, gain_std=0.1, append_rows=0)
    Blocks(cfg, blocks, 16, override=True).run_blocks()


def test_blocks_full_qwen_shape():
    # the Qwen3-8B-shaped drafter at a 2048-token context, 8 blocks anchored in
    # its second half (the response part of a training sequence): 128 block rows
    cfg = shrink(QWEN3_8B_N2048, cid=134, append_rows=0)
    rng = np.random.default_rng(134)
    anchors = sorted(rng.integers(1024, 2049, 8).tolist())
    log(f"anchored blocks, full shape, anchors {anchors}")
    Blocks(cfg, [(0, a) for a in anchors], 16).run_blocks()


def test_blocks_max_per_call():
    # 64 blocks (the most one call takes) over two sequences, anchors drawn
    # uniformly in [0, len]: up to 33 blocks share one sequence's scratch region
    rng = np.random.default_rng(7)
    ctx = (37, 300)
    blocks = [(int(s), int(rng.integers(0, ctx[s] + 1))) for s in rng.integers(0, 2, 64)]
    log(f"anchored blocks, 64 per call, {sum(1 for s, _ in blocks if s == 1)} in sequence 1")
    Blocks(small(cid=135, ctx=ctx), blocks, 16).run_blocks()
