"""Host-side cache layout helpers (runtime.DeviceCache) on CPU tensors: the
fp32 cache keeps K row-major and V transposed per head ([d][cap]); the bf16
cache keeps both per block of 32 keys, K in the attention's fragment order and
V as [d][32]; rows written with put_rows read back unchanged, sit where the C
ABI's layout puts them, and leave every other row alone."""
import numpy as np
import pytest
import torch

from block_diffusion_drafter_ctx_amd import runtime
from dflash_inputs import QWEN3_8B_N2048, shrink


def _cfg(cache_dtype):
    return shrink(QWEN3_8B_N2048, name="layout", cid=98, D=256, L=2, Hq=4, Hkv=2, d=64, F=512, V=1000, B=2,
                  ctx=(64, 20), gammas=(16,), cache_dtype=cache_dtype)


def _rows(rng, L, n, Hkv, d):
    # values exact in bf16 (a few mantissa bits), so both cache types store them unchanged
    return np.round(rng.standard_normal((L, n, Hkv, d)) * 8) / 8


@pytest.mark.parametrize("cache_dtype", ["f32", "bf16"])
def test_put_rows_round_trip_and_placement(cache_dtype):
    cfg = _cfg(cache_dtype)
    cap = 96
    c = runtime.DeviceCache(cfg, 2, cap, device="cpu")
    assert c.blocked == (cache_dtype == "bf16")
    rng = np.random.default_rng(5)
    # a range that starts mid-block and crosses two block boundaries
    lo, n = 27, 45
    k, v = _rows(rng, cfg.L, n, cfg.Hkv, cfg.d), _rows(rng, cfg.L, n, cfg.Hkv, cfg.d)
    c.put_rows(1, lo, k, v)
    k2, v2 = c.rows(1, lo, lo + n)
    assert np.array_equal(k2, k) and np.array_equal(v2, v)
    # untouched rows and the other sequence stay zero
    for part in (0, 1):
        assert not np.any(c.rows(1, 0, lo)[part]) and not np.any(c.rows(1, lo + n, cap)[part])
        assert not np.any(c.rows(0, 0, cap)[part])
    # values at the addresses the C ABI's layout gives them
    d = cfg.d
    for l, key, h, dim in [(1, lo + 9, 1, 37), (0, lo, 0, 0), (1, lo + n - 1, 0, d - 1), (0, 40, 1, 13)]:
        flat = c.v.reshape(-1)
        if c.blocked:
            off = ((((l * 2 + 1) * cfg.Hkv + h) * (cap // 32) + key // 32) * d + dim) * 32 + key % 32
        else:
            off = (((l * 2 + 1) * cfg.Hkv + h) * d + dim) * cap + key
        assert float(flat[off]) == v[l, key - lo, h, dim]
        flat = c.k.reshape(-1)
        if c.blocked:
            i = key % 32
            inblk = 512 * (((i % 8) // 4) * (d // 32) + dim // 32) + 8 * (16 * ((dim % 32) // 8) + 4 * (i // 8) + i % 4) + dim % 8
            off = (((l * 2 + 1) * cfg.Hkv + h) * (cap // 32) + key // 32) * (32 * d) + inblk
        else:
            off = (((l * 2 + 1) * cfg.Hkv + h) * cap + key) * d + dim
        assert float(flat[off]) == k[l, key - lo, h, dim]


@pytest.mark.parametrize("cache_dtype", ["f32", "bf16"])
def test_fill_random_snapshot_same_rows(cache_dtype):
    cfg = _cfg(cache_dtype)
    c = runtime.DeviceCache(cfg, 1, 64, device="cpu")
    g = torch.Generator(device="cpu")
    g.manual_seed(3)
    c.fill_random(0, 40, g)
    k, v = c.rows(0, 0, 40)
    assert np.all(np.abs(v).sum(axis=(0, 2, 3)) > 0) and np.all(np.abs(k).sum(axis=(0, 2, 3)) > 0)
    assert not np.any(c.rows(0, 40, 64)[1])            # rows past n untouched
    snap = c.snapshot(0, 40)
    assert c.same_rows(snap, 0, 40)
    c.put_rows(0, 39, np.zeros((cfg.L, 1, cfg.Hkv, cfg.d)), np.ones((cfg.L, 1, cfg.Hkv, cfg.d)))
    assert not c.same_rows(snap, 0, 40)
    assert c.same_rows(c.snapshot(0, 39), 0, 39)


@pytest.mark.parametrize("d", [64, 128])
def test_bf16_key_block_order_is_a_permutation(d):
    """The fragment order of a 32-key block is a bijection onto the block, and
    lane l of fragment f reads 8 consecutive dimensions of one key."""
    perm = runtime.k_frag_perm(d)
    assert sorted(perm.tolist()) == list(range(32 * d))
    p = perm.reshape(32, d)
    assert np.all(np.diff(p.reshape(32, d // 8, 8), axis=2) == 1)
    assert np.all(p.reshape(32, d // 8, 8)[:, :, 0] % 8 == 0)
