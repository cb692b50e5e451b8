"""Seeded input generators: determinism, storage exactness and workload shapes."""
import numpy as np

from dflash_inputs import BATCH16_RAGGED, DEEP8_B4_N8192, LONG_CTX_N32768, QWEN3_8B_N2048, TINY_F32, Inputs, bf16_round_f32, build_target_np, shrink
from dflash_inputs.gen import CHUNK


def test_seeded_and_storage_exact():
    cfg = shrink(QWEN3_8B_N2048, D=256, F=512, V=1000, L=2, ctx=(40,))
    a, b = Inputs(cfg), Inputs(cfg)
    assert np.array_equal(a.w_qkv(1), b.w_qkv(1))
    assert not np.array_equal(a.w_qkv(0), a.w_qkv(1))
    w = a.w_c()
    assert w.dtype == np.float32 and w.shape == (256, 1280)
    assert np.array_equal(w, bf16_round_f32(w.copy()))         # bf16-exact values
    assert abs(w.std() - 0.02) < 0.002
    h = a.ctx_states()
    assert len(h) == 5 and h[0].shape == (40, 256) and abs(h[0].std() - 1) < 0.1
    f32 = Inputs(TINY_F32).w_c()
    assert not np.array_equal(f32, bf16_round_f32(f32.copy()))  # fp32 workload keeps fp32


def test_chunked_generation_is_chunk_local():
    cfg = shrink(QWEN3_8B_N2048, D=2048, V=4096, ctx=(8,))
    e = Inputs(cfg).embed()              # 8M elements -> 2 chunks
    assert e.size > CHUNK
    e2 = Inputs(cfg).embed()
    assert np.array_equal(e[:16], e2[:16]) and np.array_equal(e[-16:], e2[-16:])


def test_workload_shapes():
    c4 = BATCH16_RAGGED
    assert c4.B == 16 and len(c4.ctx) == 16
    assert all(1024 <= n <= 4096 for n in c4.ctx)
    assert DEEP8_B4_N8192.gammas == (8, 16, 32)
    p = DEEP8_B4_N8192.match_probs(16)
    assert np.isclose(p[0], 0.9) and np.isclose(p[-1], 0.5)
    assert np.allclose(QWEN3_8B_N2048.match_probs(16), 0.8)


def test_block_tokens_and_targets():
    cfg = BATCH16_RAGGED
    inp = Inputs(cfg)
    t = inp.block_tokens(16)
    assert t.shape == (16, 16) and np.all(t[:, 1:] == cfg.V - 1)
    assert np.all(t[:, 0] < cfg.V - 1)
    match, r, bonus = inp.verify_draws(0, 16)
    d = np.random.default_rng(0).integers(0, cfg.V, (16, 15))
    tgt = build_target_np(d, match, r, bonus, cfg.V)
    assert tgt.shape == (16, 16)
    assert np.array_equal(tgt[:, :15] == d, match)
    assert np.all((tgt >= 0) & (tgt < cfg.V))


def test_sampling_uniforms_open_and_exact():
    cfg = shrink(QWEN3_8B_N2048, V=5000, B=2)
    inp = Inputs(cfg)
    g, a, e = inp.sample_uniforms(0, 16)
    assert g.shape == (2, 15, 5000) and a.shape == (2, 15) and e.shape == (2, 5000)
    for u in (g, a, e):
        assert u.dtype == np.float32 and u.min() > 0.0 and u.max() < 1.0
        k = u.astype(np.float64) * 2.0 ** 24               # odd integers: exact in float32
        assert np.array_equal(k, np.round(k)) and np.all(np.round(k) % 2 == 1)
    g2, _, _ = Inputs(cfg).sample_uniforms(0, 16)
    assert np.array_equal(g, g2)
    assert not np.array_equal(g, inp.sample_uniforms(1, 16)[0])
    assert abs(g.mean() - 0.5) < 0.01


def test_synthetic_target_logits():
    from dflash_inputs import build_target_logits_np
    cfg = shrink(QWEN3_8B_N2048, V=3000, B=2)
    inp = Inputs(cfg)
    z = inp.synthetic_logits(0, 16, 1.28)
    nz = inp.target_noise(0, 16)
    t = build_target_logits_np(z, nz)
    assert t.shape == (2, 16, 3000) and abs(z.std() - 1.28) < 0.02
    assert np.allclose(t[:, :15] - z, 0.5 * nz[:, :15], atol=1e-6)
    assert np.array_equal(t[:, 15], nz[:, 15])
    ids = inp.random_ids(0, 16)
    assert ids.shape == (2, 15) and ids.min() >= 0 and ids.max() < 3000


def test_runtime_tap_layers_match_the_oracle():
    # the product side's tap-layer rule (integer arithmetic) against the oracle's
    from block_diffusion_drafter_ctx_amd.runtime import tap_layers
    from oracle import dflash_oracle as O
    for L_t in range(4, 129):
        for n in (2, 3, 4, 5, 6, 8):
            if L_t - 3 >= 1:
                assert tap_layers(L_t, n) == O.tap_layers(L_t, n), (L_t, n)
    assert tap_layers(36) == [1, 9, 17, 25, 33]
