"""dflash_draft_forward_noalloc (the pass with its workspace in the library's
static device array) against dflash_draft_forward with a caller workspace.

Both run the same kernels on the same inputs, so the final states, the block
K/V rows they store and the context rows they leave alone must agree bit for
bit.  Each case makes two no-allocation calls in a row, the second with a
smaller block, so the second pass runs over scratch the first one left behind.
"""
import numpy as np
import pytest
import torch

from block_diffusion_drafter_ctx_amd import binding as B
from block_diffusion_drafter_ctx_amd.runtime import DeviceDrafter, upload
from dflash_inputs import QWEN3_8B_N2048, Inputs, shrink
from tests.parity_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("the no-allocation tests need a gfx950 GPU")
    B.load()


def _setup(cfg, gmax):
    inp = Inputs(cfg)
    dr = DeviceDrafter(cfg, inp)
    cap = (max(cfg.ctx) + gmax + 31) // 32 * 32
    cache = dr.cache(cfg.B, cap)
    dr.ensure_workspace(cfg.B, gmax, max(cfg.n_ctx_total, 1))
    states = [upload(h, cfg) for h in inp.ctx_states()]
    H_t = dr.context_buffer(cfg.n_ctx_total)
    dr.fuse(states, cfg.n_ctx_total, H_t)
    dr.inject(H_t, list(cfg.ctx), cache)
    torch.cuda.synchronize()
    return inp, dr, cache


def _pass(dr, cache, tok, ov, gamma, noalloc):
    cfg = dr.cfg
    h = torch.full((cfg.B, gamma, cfg.D), float("nan"), dtype=torch.float32, device="cuda")
    if noalloc:
        B.draft_forward_noalloc(dr.dims, dr.weights, cache.struct, 0 if tok is None else tok.data_ptr(),
                                0 if ov is None else ov.data_ptr(), gamma, h.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    else:
        dr.draft(cache, tok, ov, gamma, h)
    torch.cuda.synchronize()
    lens = cache.len_list()
    blk = [cache.rows(b, lens[b], lens[b] + gamma) for b in range(cfg.B)]
    return h.clone(), blk


def _compare(dr, cache, inp, gammas, override):
    cfg = dr.cfg
    lens = cache.len_list()
    snap = [cache.snapshot(b, lens[b]) for b in range(cfg.B)]
    for gamma in gammas:                      # second call: a smaller block
        tok = torch.from_numpy(inp.block_tokens(gamma)).cuda()
        ov = torch.from_numpy(inp.embed_override(gamma)).cuda() if override else None
        h_ref, blk_ref = _pass(dr, cache, tok, ov, gamma, noalloc=False)
        h_got, blk_got = _pass(dr, cache, tok, ov, gamma, noalloc=True)
        assert torch.isfinite(h_got).all()
        assert torch.equal(h_got, h_ref), f"gamma {gamma}: final states differ"
        for b in range(cfg.B):
            assert np.array_equal(blk_got[b][0], blk_ref[b][0]) and np.array_equal(blk_got[b][1], blk_ref[b][1])
            assert cache.same_rows(snap[b], b, lens[b]), "context rows changed"
        d_ref = torch.empty(cfg.B, gamma - 1, dtype=torch.int32, device="cuda")
        d_got = torch.empty_like(d_ref)
        dr.argmax_accept(B.ARGMAX, h_ref, cfg.B, gamma, d_ref)
        dr.argmax_accept(B.ARGMAX, h_got, cfg.B, gamma, d_got)
        torch.cuda.synchronize()
        assert torch.equal(d_got, d_ref)
        log(f"no-alloc {cfg.name}: gamma {gamma} bit-identical to the workspace call")


def test_noalloc_small_two_calls():
    cfg = shrink(QWEN3_8B_N2048, name="noalloc_small", cid=601, D=512, L=2, Hq=8, Hkv=2, d=128, F=1536, V=1000,
                 B=3, ctx=(37, 300, 1), gain_std=0.1)
    inp, dr, cache = _setup(cfg, 16)
    _compare(dr, cache, inp, [16, 5], override=True)


def test_noalloc_small_bf16_cache_two_calls():
    cfg = shrink(QWEN3_8B_N2048, name="noalloc_small_bf16", cid=602, D=512, L=2, Hq=8, Hkv=2, d=128, F=1536,
                 V=1000, B=2, ctx=(130, 64), gain_std=0.1, cache_dtype="bf16")
    inp, dr, cache = _setup(cfg, 16)
    _compare(dr, cache, inp, [16, 8], override=False)


@pytest.mark.timeout(600)
def test_noalloc_qwen3_8b_shape_two_calls():
    cfg = QWEN3_8B_N2048
    inp, dr, cache = _setup(cfg, 16)
    _compare(dr, cache, inp, [16, 8], override=False)


def test_noalloc_refuses_a_pass_beyond_its_scratch():
    # 64 sequences of 33 rows at D = 2048 need far more than the static array:
    # refused on the host, nothing written
    cfg = shrink(QWEN3_8B_N2048, name="noalloc_big", cid=603, D=2048, L=1, Hq=16, Hkv=4, d=128, F=4096, V=1000,
                 B=64, ctx=(8,) * 64)
    inp = Inputs(cfg)
    dr = DeviceDrafter(cfg, inp)
    cache = dr.cache(cfg.B, 64)
    h = torch.full((cfg.B, 33, cfg.D), 7.0, device="cuda")
    tok = torch.from_numpy(inp.block_tokens(33)).cuda()
    with pytest.raises(B.DFlashError) as e:
        B.draft_forward_noalloc(dr.dims, dr.weights, cache.struct, tok.data_ptr(), 0, 33, h.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    assert e.value.status == B.ERR_WORKSPACE and "no-allocation" in B.last_error()
    torch.cuda.synchronize()
    assert torch.all(h == 7.0)
