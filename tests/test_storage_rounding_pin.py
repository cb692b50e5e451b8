"""What two correct evaluations of a bf16 cache disagree on (CPU, full size).

With a bf16 H_t / KV cache every stored value is rounded once to bfloat16
(round to nearest even).  An fp32 implementation accumulates the fused
projection and the K/V projections in float32 before that rounding; the oracle
accumulates in float64.  Where the exact value lies within the float32
accumulation error of a bf16 rounding boundary the two store neighbouring bf16
numbers.  This test measures, at the Qwen3-8B drafter shape (D = 4096,
5 layers, 32/8 heads of 128, FFN 12288, V = 151936, a 2048-row context), how
far apart such flips put two correct evaluations, by running the oracle's
drafter forward (float64) over two caches built from the same seeded inputs:
one whose stored values were accumulated in float64 (the oracle itself), one
whose stored values were accumulated in float32 (numpy's single-precision
BLAS).  It pins the readings the GPU parity tests use for a bf16 cache:

  * stored tensors may differ from the oracle beyond the max-abs tolerance
    only by exactly one bf16 ulp, on a small share of elements (here ~0.6%
    of K/V elements and ~0.02% of H_t elements differ at all; one-ulp steps
    beyond 2e-2 stay under 0.1%);
  * the logits of the two evaluations stay within a few 1e-3 of each other,
    so the argmax rule of the pages' tolerance (agreement wherever the
    oracle's top-2 gap is >= 1e-3) is held to as stated, with no wider
    exclusion for a bf16 cache.
"""
import numpy as np
import pytest

from dflash_inputs import QWEN3_8B_N2048, Inputs, shrink
from oracle import dflash_oracle as O

NSETS = 8          # independent blocks of 16 distinct rows over the same cache: 120 LM-head rows


def bf16_ulp(x):
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 7)


def stored_differences(a, b):
    """Share of elements that differ, and share that differ by more than the
    max-abs tolerance 2e-2; asserts that every difference beyond 2e-2 is
    exactly one bf16 ulp (of the smaller value) -- the stored-tensor rule of
    the GPU parity tests."""
    diff = a != b
    step = np.abs(a - b)
    over = step > 2e-2
    if over.any():
        ulp = np.minimum(bf16_ulp(a[over]), bf16_ulp(b[over]))
        assert np.all(step[over] == ulp), "a stored difference beyond 2e-2 that is not one bf16 ulp"
    return float(diff.mean()), float(over.mean())


@pytest.fixture(scope="module")
def two_evaluations():
    cfg = shrink(QWEN3_8B_N2048, cid=203, cache_dtype="bf16", B=NSETS)
    inp = Inputs(cfg)
    states = inp.ctx_states()
    wc, gc = inp.w_c(), inp.g_c()
    # float64-accumulated storage: the oracle
    ht64 = O.fuse_context(states, wc, gc, cfg.eps, "bf16")
    # float32-accumulated storage: the same definition, single-precision BLAS
    u32 = np.concatenate(states, axis=1) @ wc.T
    ms = np.mean(u32 * u32, axis=-1, keepdims=True, dtype=np.float32)
    ht32 = O.to_bf16((gc * (u32 / np.sqrt(ms + np.float32(cfg.eps)))).astype(np.float32))
    del u32, states
    c64 = O.OracleCache(cfg.L, NSETS, cfg.Hkv, cfg.d)
    c32 = O.OracleCache(cfg.L, NSETS, cfg.Hkv, cfg.d)
    kv_flips = []
    layers = []
    f = lambda a: np.asarray(a, dtype=np.float64)  # noqa: E731
    for l in range(cfg.L):
        wq = inp.w_qkv(l)
        k64, v64 = O.inject_kv(ht64, wq, cfg.Hq, cfg.Hkv, cfg.d, "bf16")
        _, wk, wv = O.split_qkv(wq, cfg.Hq, cfg.Hkv, cfg.d)
        h32 = ht32.astype(np.float32)
        k32 = O.to_bf16(h32 @ wk.T).reshape(k64.shape)
        v32 = O.to_bf16(h32 @ wv.T).reshape(v64.shape)
        kv_flips.append((stored_differences(k64, k32), stored_differences(v64, v32)))
        for b in range(NSETS):      # every block sees the same context rows
            c64.append(l, b, k64, v64)
            c32.append(l, b, k32, v32)
        layers.append(dict(w_qkv=f(wq), w_o=f(inp.w_o(l)), w_gateup=f(inp.w_gateup(l)), w_down=f(inp.w_down(l)),
                           g_attn=f(inp.g_attn(l)), g_ffn=f(inp.g_ffn(l))))
    ov = inp.embed_override(16)
    gf = f(inp.g_final())
    hf64, bkv64 = O.draft_forward(cfg, layers, gf, c64, 16, override=ov, storage="bf16")
    hf32, bkv32 = O.draft_forward(cfg, layers, gf, c32, 16, override=ov, storage="bf16")
    # the block's own K/V rows of every layer: two forwards of one definition
    # whose inputs differ only through the bf16 flips of their caches
    block_flips = [(stored_differences(k64, k32), stored_differences(v64, v32))
                   for (k64, v64), (k32, v32) in zip(bkv64, bkv32)]
    del layers, c64, c32
    E = f(inp.embed())
    d64, gap64, z64 = O.lm_head_argmax(hf64, E)
    d32, _, z32 = O.lm_head_argmax(hf32, E)
    return dict(ht_flips=stored_differences(ht64, ht32), kv_flips=kv_flips, block_flips=block_flips, d64=d64,
                d32=d32, gap64=gap64, drift=np.abs(z64 - z32))


def test_stored_values_differ_by_one_ulp_at_most(two_evaluations):
    r = two_evaluations
    # H_t: an fp32 sum over 5D = 20480 terms, then RMSNorm (measured: 0.02% of
    # elements differ, none by more than 2e-2)
    share, over = r["ht_flips"]
    assert 0.0 < share < 1e-3 and over <= 1e-3, r["ht_flips"]
    # K/V: fp32 sums over D = 4096 terms of bf16 products of a (slightly
    # different) H_t; a few tenths of a percent of elements differ in every
    # layer (measured ~0.6%), and one-ulp flips beyond 2e-2 stay under 0.1%
    for (sk, ok), (sv, ov) in r["kv_flips"]:
        assert 1e-3 < sk < 2e-2 and 1e-3 < sv < 2e-2, r["kv_flips"]
        assert ok <= 1e-3 and ov <= 1e-3, r["kv_flips"]


def test_logit_drift_stays_below_a_few_thousandths(two_evaluations):
    drift = two_evaluations["drift"]
    # the flips move the logits, but by a few 1e-3 at most (measured 2.1e-3)
    assert 1e-4 < float(drift.max()) < 5e-3, float(drift.max())
    assert float(np.quantile(drift, 0.99)) < 1.5e-3


def test_argmax_agrees_above_the_stated_gap(two_evaluations):
    r = two_evaluations
    sure = r["gap64"] >= 1e-3
    assert sure.sum() >= 100
    assert np.array_equal(r["d64"][sure], r["d32"][sure])


def test_block_kv_flips_grow_with_depth(two_evaluations):
    """The block's K/V rows are rounded from activations that carry every
    earlier layer's drift: layer 0's inputs are identical in both evaluations
    (no flips), deeper layers' differ, and their one-ulp flips beyond 2e-2
    appear and grow with depth.  (Measured here from the caches' flips alone;
    an fp32 forward adds its own accumulation drift on top.)"""
    fl = two_evaluations["block_flips"]
    print("block K/V flip shares per layer (all, beyond 2e-2):", fl)
    (k0, _), (v0, _) = fl[0]
    assert k0 == 0.0 and v0 == 0.0
    deep = [max(k[0], v[0]) for k, v in fl[1:]]
    assert all(x > 0.0 for x in deep)
    assert max(k[1] + v[1] for k, v in fl[2:]) >= max(k[1] + v[1] for k, v in fl[1:2])
