"""HIP path against the CPU oracle on seeded inputs (needs an MI355X)."""
import numpy as np
import pytest
import torch

from block_diffusion_drafter_ctx_amd import binding as B
from block_diffusion_drafter_ctx_amd.runtime import upload
from dflash_inputs import BATCH16_RAGGED, DEEP8_B4_N8192, LONG_CTX_N32768, QWEN3_8B_N2048, TINY_F32, Inputs, shrink
from tests.parity_util import Workload, close, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU parity tests need a gfx950 GPU")
    B.load()
    log(f"library {B.version()} on {torch.cuda.get_device_name(0)}")


def small(**kw):
    """Several weight tiles, a ragged vocabulary tail, GQA 4, ragged context."""
    base = dict(name="small_bf16", cid=101, D=512, L=2, Hq=8, Hkv=2, d=128, F=1536, V=1000, B=3,
                ctx=(37, 300, 1), gammas=(16,), gain_std=0.1, iters=2)
    base.update(kw)
    return shrink(QWEN3_8B_N2048, **base)


def test_small_bf16_tokens():
    log("small bf16, token embeddings, 2 iterations")
    Workload(small(), 16, 2).run()


def test_small_bf16_override():
    log("small bf16, distinct override rows")
    Workload(small(cid=102), 16, 1, override=True).run()


def test_small_bf16_cache():
    log("small bf16 weights with a bf16 H_t / KV cache")
    Workload(small(cid=108, cache_dtype="bf16"), 16, 2, override=True).run()


@pytest.mark.parametrize("gamma", [2, 5, 33])
def test_small_bf16_gamma_edges(gamma):
    log(f"small bf16, gamma={gamma}")
    Workload(small(cid=103, gammas=(gamma,)), gamma, 1, override=True).run()


@pytest.mark.parametrize("gamma", [2, 5, 17, 33])
def test_small_bf16_cache_gamma_edges(gamma):
    # bf16 cache: G * gamma query rows per KV head of 8, 20 (two wave groups),
    # 68 (one group of eight waves) and 132 (two row groups)
    log(f"small bf16, bf16 cache, gamma={gamma}")
    Workload(small(cid=109, gammas=(gamma,), cache_dtype="bf16"), gamma, 1, override=True).run()


def test_small_head64_bf16_cache():
    log("small bf16, head_dim 64, bf16 cache, a sequence with no context rows")
    cfg = small(cid=110, d=64, Hq=4, Hkv=4, ctx=(0, 70), B=2, V=777 * 2, cache_dtype="bf16")
    Workload(cfg, 8, 1, override=True).run()


def test_small_head64_empty_context():
    log("small bf16, head_dim 64, a sequence with no context rows")
    cfg = small(cid=104, d=64, Hq=4, Hkv=4, ctx=(0, 70), B=2, V=777 * 2)
    Workload(cfg, 8, 1, override=True).run()


def test_register_k_shapes():
    # one sequence of gamma = 16: 16 block rows and 15 LM-head rows, D = 2048
    # (4 k-steps per wave), a gate/up weight of 2F = 16384 rows and an odd
    # vocabulary (ragged last tile) take the register-K GEMM, with the LM-head
    # top-2 and SwiGLU epilogues; the short weights take its split-K form
    log("register-K shapes: D=2048, 2F=16384, V=20001, batch 1")
    cfg = small(cid=109, D=2048, L=1, Hq=16, Hkv=4, d=128, F=8192, V=20001, B=1, ctx=(256,), iters=2)
    Workload(cfg, 16, 2, override=True).run()
    Workload(shrink(cfg, cid=110), 16, 1).run()
    # partial row blocks: 5 block rows / 4 LM-head rows (rows past M masked),
    # and a 2-sequence batch of 7 (14 rows) through the same kernels
    Workload(shrink(cfg, cid=111, gammas=(5,)), 5, 1, override=True).run()
    Workload(shrink(cfg, cid=112, B=2, ctx=(40, 300), gammas=(7,)), 7, 1, override=True).run()
    # F = 6144: the down projection (K = 6144) takes six k-steps per wave (4
    # splits on 256 workgroups rather than 6 on 252), and gate/up (2F = 12288
    # rows, below the tall form) the split-K form with the separate SwiGLU;
    # 16, 5 and 14 block rows
    log("register-K shapes: F=6144 (six k-steps per wave on the down projection)")
    cfg6 = shrink(cfg, cid=140, F=6144)
    Workload(cfg6, 16, 1).run()
    Workload(shrink(cfg6, cid=141, gammas=(5,)), 5, 1, override=True).run()
    Workload(shrink(cfg6, cid=142, B=2, ctx=(40, 300), gammas=(7,)), 7, 1, override=True).run()


def test_register_k_row_chunks(monkeypatch):
    # more than 16 activation rows on the register-K kernel, one workgroup per
    # 16-row chunk.  By default the tall forms take up to 32 rows: 2 sequences
    # of 13 give 26 block rows (gate/up with SwiGLU) and 24 LM-head rows (top-2),
    # two chunks, the second partial.
    log("register-K row chunks: D=2048, 2F=16384, V=20001, 26 block / 24 LM-head rows")
    cfg = small(cid=113, D=2048, L=1, Hq=16, Hkv=4, d=128, F=8192, V=20001, B=2, ctx=(256, 7), gammas=(13,),
                iters=2)
    Workload(cfg, 13, 2, override=True).run()
    # every form allowed up to 128 rows: 39 block rows and 36 LM-head rows
    # (three chunks), 48 appended rows through the fuse and inject GEMMs, and 8
    # sequences of 16 (128 block rows, 120 LM-head rows: eight chunks)
    monkeypatch.setenv("DFLASH_RK_MAX_ROWS", "128")
    log("register-K row chunks up to 128 rows: 39 / 36 / 48 rows, then 128 / 120")
    Workload(shrink(cfg, cid=115, B=3, ctx=(256, 40, 7)), 13, 2, override=True).run()
    cfg8 = shrink(cfg, cid=114, B=8, ctx=(256, 40, 7, 0, 100, 31, 64, 200), gammas=(16,), iters=1)
    Workload(cfg8, 16, 1).run()


def test_tile_order_bit_identical(monkeypatch):
    # the tiled GEMM's XCD-grouped launch order only moves tiles between
    # workgroups: 5 sequences of 16 (80 block rows, 75 LM-head rows, tiled
    # GEMMs with hi/lo planes) give the same bits in grid order
    cfg = small(cid=116, B=5, ctx=(37, 300, 1, 64, 129))
    w = Workload(cfg, 16, 1, override=True)
    w.ingest(w.inp.ctx_states(), list(cfg.ctx), "context")
    ov = torch.from_numpy(w.inp.embed_override(16)).cuda()
    outs = []
    for order in ("1", "2"):
        monkeypatch.setenv("DFLASH_TILE_XCD", order)
        h = torch.empty(cfg.B, 16, cfg.D, device="cuda")
        w.dr.draft(w.cache, None, ov, 16, h)
        d = torch.empty(cfg.B, 15, dtype=torch.int32, device="cuda")
        z = torch.empty(cfg.B, 15, cfg.V, device="cuda")
        w.dr.argmax_accept(B.ARGMAX, h, cfg.B, 16, d, logits=z)
        torch.cuda.synchronize()
        outs.append((h.clone(), d.clone(), z.clone()))
    log("tile order: XCD-grouped and grid order agree bit for bit")
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_tiny_f32():
    cfg = TINY_F32
    log("tiny_f32: tiny fp32 drafter")
    Workload(cfg, cfg.gamma, 3).run()


def test_tiny_f32_override():
    cfg = shrink(TINY_F32, cid=105, gain_std=0.1)
    Workload(cfg, cfg.gamma, 1, override=True).run()


def test_determinism_and_untouched_context():
    cfg = small(cid=106)
    w = Workload(cfg, 16, 1, override=True)
    w.ingest(w.inp.ctx_states(), list(cfg.ctx), "context")
    lens = w.cache.len_list()
    snap = [w.cache.snapshot(b, lens[b]) for b in range(cfg.B)]
    tok = torch.from_numpy(w.inp.block_tokens(16)).cuda()
    outs = []
    for _ in range(2):
        h = torch.empty(cfg.B, 16, cfg.D, device="cuda")
        w.dr.draft(w.cache, tok, None, 16, h)
        d = torch.empty(cfg.B, 15, dtype=torch.int32, device="cuda")
        w.dr.argmax_accept(B.ARGMAX, h, cfg.B, 16, d)
        torch.cuda.synchronize()
        outs.append((h.clone(), d.clone(), w.cache.k.clone(), w.cache.v.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(outs[0][2], outs[1][2]) and torch.equal(outs[0][3], outs[1][3])
    for b in range(cfg.B):
        assert w.cache.same_rows(snap[b], b, lens[b])
    # fuse + inject again from scratch gives bit-identical cache rows
    c2 = w.dr.cache(cfg.B, w.cache.cap)
    h_dev = [upload(h, cfg) for h in w.inp.ctx_states()]
    Ht = w.dr.context_buffer(cfg.n_ctx_total)
    w.dr.fuse(h_dev, cfg.n_ctx_total, Ht)
    w.dr.inject(Ht, list(cfg.ctx), c2)
    torch.cuda.synchronize()
    for b in range(cfg.B):
        assert c2.same_rows(snap[b], b, lens[b])
    assert c2.len_dev.cpu().tolist() == lens


def test_errors_enqueue_nothing():
    cfg = small(cid=107)
    w = Workload(cfg, 16, 1)
    w.ingest(w.inp.ctx_states(), list(cfg.ctx), "context")
    k0 = w.cache.k.clone()
    lens = w.cache.len_list()
    w.cache.set_lens([w.cache.cap - 3] + lens[1:])
    h = torch.full((cfg.B, 16, cfg.D), 7.0, device="cuda")
    tok = torch.from_numpy(w.inp.block_tokens(16)).cuda()
    with pytest.raises(B.DFlashError) as e:
        w.dr.draft(w.cache, tok, None, 16, h)
    assert e.value.status == B.ERR_CAPACITY
    torch.cuda.synchronize()
    assert torch.all(h == 7.0) and torch.equal(w.cache.k, k0)
    w.cache.set_lens(lens)


@pytest.mark.timeout(900)
def test_qwen3_8b_n2048():
    cfg = QWEN3_8B_N2048
    log("qwen3_8b_shape_n2048 full size (N=2048), 8 iterations, each appending 16 rows")
    Workload(cfg, 16, 8).run()


@pytest.mark.timeout(900)
def test_qwen3_8b_n2048_override():
    cfg = shrink(QWEN3_8B_N2048, cid=202)
    log("qwen3_8b_shape_n2048 full size with distinct block rows (argmax on 15 different rows)")
    Workload(cfg, 16, 1, override=True).run()


@pytest.mark.timeout(900)
def test_qwen3_8b_n2048_bf16_cache():
    cfg = shrink(QWEN3_8B_N2048, cid=203, cache_dtype="bf16")
    log("qwen3_8b_shape_n2048 full size, bf16 H_t / KV cache, distinct block rows, 8 iterations + appends")
    Workload(cfg, 16, 8, override=True).run()


def test_bf16_storage_rounding_is_rne():
    """Cache K values that are exact fp32 sums on and around bf16 ties must be
    stored with round-to-nearest-even, bit for bit (checked against the oracle's
    rounding)."""
    import ctypes
    from oracle import dflash_oracle as O
    D, d, Hq, Hkv, L = 64, 64, 1, 1, 1
    dims = B.Dims(D=D, L=L, Hq=Hq, Hkv=Hkv, head_dim=d, F=64, V=8, n_tgt_layers=5, mask_id=7,
                  rms_eps=1e-6, dtype=B.BF16, cache_dtype=B.BF16)
    base = [1.0, 2.0 ** -9, 2.0 ** -8, 3 * 2.0 ** -8, 2.0 ** -7, 3 * 2.0 ** -9, -1.0, -(2.0 ** -8)]
    H = np.zeros((4, D), dtype=np.float32)
    for t in range(4):
        H[t, :8] = np.array(base, dtype=np.float32) * (2.0 ** t)
    # key column c = H[c % 8 pair]: sums of two bf16 entries, exact in fp32
    pairs = [(0, 1), (0, 2), (0, 3), (0, 4), (0, 5), (6, 7), (6, 2), (1, 2)]
    w = np.zeros(((Hq + 2 * Hkv) * d, D), dtype=np.float32)
    for c in range(d):
        a, b = pairs[c % 8]
        w[Hq * d + c, a] = 1.0
        w[Hq * d + c, b] = 1.0
        w[(Hq + Hkv) * d + c, a] = 1.0
        w[(Hq + Hkv) * d + c, b] = -1.0
    Ht = torch.from_numpy(H).cuda().to(torch.bfloat16)
    wq = torch.from_numpy(w).cuda().to(torch.bfloat16)
    kc = torch.zeros(L, 1, Hkv, 1, 32 * d, dtype=torch.bfloat16, device="cuda")  # bf16 K: [cap/32][32 d], fragment order
    vc = torch.zeros(L, 1, Hkv, 1, d, 32, dtype=torch.bfloat16, device="cuda")   # bf16 V: [cap/32][d][32]
    lens = (ctypes.c_int32 * 1)(0)
    cache = B.KVCache(k=kc.data_ptr(), v=vc.data_ptr(), B=1, cap=32, len=ctypes.cast(lens, ctypes.POINTER(ctypes.c_int32)))
    wts = B.Weights(w_qkv=wq.data_ptr())
    nbytes = B.workspace_size(dims, 1, 2, 4)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    B.inject_kv(dims, wts, Ht.data_ptr(), [4], cache, ws.data_ptr(), nbytes, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert lens[0] == 4
    exact_k = H.astype(np.float64) @ w[Hq * d:(Hq + Hkv) * d].astype(np.float64).T     # [4, d]
    exact_v = H.astype(np.float64) @ w[(Hq + Hkv) * d:].astype(np.float64).T
    from block_diffusion_drafter_ctx_amd.runtime import k_frag_perm
    got_k = kc[0, 0, 0, 0].float().cpu().numpy()[k_frag_perm(d)].reshape(32, d)[:4]
    got_v = vc[0, 0, 0, 0, :, :4].float().cpu().numpy().T
    assert np.array_equal(got_k, O.to_bf16(exact_k)), (got_k[0, :8], O.to_bf16(exact_k)[0, :8])
    assert np.array_equal(got_v, O.to_bf16(exact_v))
    # the test really exercises ties: some exact values are not bf16 numbers
    assert not np.array_equal(exact_k, O.to_bf16(exact_k))


@pytest.mark.timeout(1200)
def test_long_ctx_n32768():
    cfg = LONG_CTX_N32768
    log("long_ctx_n32768 full size: 32768-row context, 8 iterations, each appending 16 rows")
    Workload(cfg, 16, 8).run()


@pytest.mark.timeout(1200)
def test_long_ctx_n32768_bf16_cache():
    cfg = shrink(LONG_CTX_N32768, cid=303, cache_dtype="bf16")
    log("long_ctx_n32768 full size with a bf16 H_t / KV cache: 32768-row context, 8 iterations + appends")
    Workload(cfg, 16, 8).run()


@pytest.mark.timeout(1200)
def test_batch16_ragged():
    cfg = BATCH16_RAGGED
    log(f"batch16_ragged full size: 16 ragged sequences {list(cfg.ctx)}, 8 iterations, each appending 16 rows")
    Workload(cfg, 16, 8).run()


@pytest.mark.timeout(1200)
def test_batch16_ragged_bf16_cache():
    # the bench's batch16 loop runs on a bf16 cache: 16 sequences' block-major
    # V rows, key ranges planned across all of them
    # (distinct block rows: with mask rows, 15 identical rows of a block round
    # together, so one near-tie flips 15 elements of the block K/V at once)
    cfg = shrink(BATCH16_RAGGED, cid=304, cache_dtype="bf16")
    log(f"batch16_ragged full size, bf16 H_t / KV cache {list(cfg.ctx)}, distinct block rows, 4 iterations + appends")
    Workload(cfg, 16, 4, override=True).run()


@pytest.mark.timeout(1200)
def test_deep8_b4_n8192_bf16_cache_gamma_sweep():
    cfg = shrink(DEEP8_B4_N8192, cid=305, cache_dtype="bf16")
    log("deep8_b4_n8192 full size, bf16 H_t / KV cache, distinct block rows: gamma 8 / 16 / 32 on one cache")
    w = Workload(cfg, max(cfg.gammas), 1, override=True)
    w.run_gammas(list(cfg.gammas))


@pytest.mark.timeout(1200)
def test_deep8_b4_n8192_gamma_sweep():
    cfg = DEEP8_B4_N8192
    log("deep8_b4_n8192 full size: 8 layers, 4 x 8192 context, gamma 8 / 16 / 32 on one cache")
    w = Workload(cfg, max(cfg.gammas), 1)
    w.run_gammas(list(cfg.gammas))
