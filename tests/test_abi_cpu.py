"""The C-ABI library without a GPU: it loads, exports every declared symbol,
and rejects bad arguments on the host with the documented status before any
HIP call (no compute call is made here)."""
import ctypes
import re
import os

import pytest

from block_diffusion_drafter_ctx_amd import binding as B

HDR = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "dflash.h")


def _dims(**kw):
    d = dict(D=256, L=2, Hq=4, Hkv=2, head_dim=64, F=512, V=1000, n_tgt_layers=5, mask_id=999,
             rms_eps=1e-6, dtype=B.BF16, cache_dtype=B.F32)
    d.update(kw)
    return B.Dims(**d)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libdflash.so is not built (run __graft_entry__.build())")
    return B.load()


def test_exports_every_declared_symbol(lib):
    declared = set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", open(HDR).read()))
    assert declared == set(B.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    assert "gfx950" in B.version()


def test_workspace_size_pure_host(lib):
    n = B.workspace_size(_dims(), 1, 16, 128)
    assert n > 0
    big = B.workspace_size(_dims(D=4096, F=12288, Hq=32, Hkv=8, head_dim=128, V=151936, L=5), 16, 16, 65536)
    assert big > n


@pytest.mark.parametrize("bad", [
    dict(D=100), dict(D=0), dict(F=100), dict(head_dim=96), dict(Hq=6, Hkv=4), dict(L=0),
    dict(n_tgt_layers=0), dict(n_tgt_layers=9), dict(V=1), dict(mask_id=1000), dict(mask_id=-1),
    dict(rms_eps=0.0), dict(rms_eps=float("nan")), dict(dtype=7), dict(cache_dtype=3),
    dict(dtype=B.F32, cache_dtype=B.BF16),
])
def test_bad_dims_rejected(lib, bad):
    with pytest.raises(B.DFlashError) as e:
        B.workspace_size(_dims(**bad), 1, 16, 16)
    assert e.value.status == B.ERR_INVALID_ARG
    assert B.last_error()


@pytest.mark.parametrize("gamma", [0, 1, 34, 100])
def test_bad_gamma(lib, gamma):
    with pytest.raises(B.DFlashError) as e:
        B.workspace_size(_dims(), 1, gamma, 16)
    assert e.value.status == B.ERR_INVALID_ARG


def _cache(Bn=2, cap=64, lens=(0, 0), k=0x10000, v=0x20000, len_dev=0):
    arr = (ctypes.c_int32 * Bn)(*lens)
    c = B.KVCache(k=k, v=v, B=Bn, cap=cap, len=ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)), len_dev=len_dev)
    c._keep = arr
    return c


def test_inject_capacity_checked_before_any_work(lib):
    c = _cache(lens=(60, 0))
    w = B.Weights(w_qkv=0x1000)
    with pytest.raises(B.DFlashError) as e:
        B.inject_kv(_dims(), w, 0x3000, [5, 1], c, 0, 0)
    assert e.value.status == B.ERR_CAPACITY
    assert list(c._keep) == [60, 0]          # len untouched


def test_draft_capacity_and_nulls(lib):
    w = B.Weights(w_qkv=0x1000, w_o=0x1000, w_gateup=0x1000, w_down=0x1000, g_attn=0x1000, g_ffn=0x1000,
                  g_final=0x1000, embed=0x1000, lm_head=0x1000)
    with pytest.raises(B.DFlashError) as e:
        B.draft_forward(_dims(), w, _cache(lens=(50, 0)), 0x4000, None, 16, 0x5000, 0x100000, 1 << 30)
    assert e.value.status == B.ERR_CAPACITY
    with pytest.raises(B.DFlashError) as e:
        B.draft_forward(_dims(), w, _cache(), None, None, 16, 0x5000, 0x100000, 1 << 30)
    assert e.value.status == B.ERR_INVALID_ARG
    w2 = B.Weights(w_qkv=0x1000)
    with pytest.raises(B.DFlashError) as e:
        B.draft_forward(_dims(), w2, _cache(), 0x4000, None, 16, 0x5000, 0x100000, 1 << 30)
    assert e.value.status == B.ERR_INVALID_ARG


def test_bf16_cache_shape_limit_checked_before_any_work(lib):
    # the bf16-cache attention addresses one head's K or V with 32-bit byte
    # offsets: cap * head_dim * 2 >= 2^32 is refused on the host, before any
    # launch (and before the device is even looked at)
    w = B.Weights(w_qkv=0x1000, w_o=0x1000, w_gateup=0x1000, w_down=0x1000, g_attn=0x1000, g_ffn=0x1000,
                  g_final=0x1000, embed=0x1000, lm_head=0x1000)
    cap = (1 << 32) // (64 * 2)                 # exactly 2^32 bytes per head at head_dim 64
    with pytest.raises(B.DFlashError) as e:
        B.draft_forward(_dims(cache_dtype=B.BF16), w, _cache(cap=cap), 0x4000, None, 16, 0x5000, 0x100000, 1 << 30)
    assert e.value.status == B.ERR_UNSUPPORTED
    with pytest.raises(B.DFlashError) as e:
        B.draft_forward_ragged(_dims(cache_dtype=B.BF16), w, _cache(cap=cap), 0x4000, None, [16, 8], 0x5000,
                               0x100000, 1 << 30)
    assert e.value.status == B.ERR_UNSUPPORTED
    with pytest.raises(B.DFlashError) as e:
        B.draft_forward_blocks(_dims(cache_dtype=B.BF16), w, _cache(cap=cap), [0], [0], 16, 0x4000, None, 0x5000,
                               0x100000, 1 << 30)
    assert e.value.status == B.ERR_UNSUPPORTED
    # one 32-row step below the limit passes this check (and then fails on the
    # missing device, not on the shape)
    with pytest.raises(B.DFlashError) as e:
        B.draft_forward(_dims(cache_dtype=B.BF16), w, _cache(cap=cap - 32), 0x4000, None, 16, 0x5000, 0x100000,
                        1 << 30)
    assert e.value.status != B.ERR_UNSUPPORTED or "gfx950" in B.last_error()


def test_noalloc_refuses_passes_beyond_its_scratch(lib):
    # the size check is host-side and comes before any device call: a pass
    # that fits goes on to look for the device (absent here), one that does
    # not is refused with DFLASH_ERR_WORKSPACE
    qwen = dict(D=4096, L=5, Hq=32, Hkv=8, head_dim=128, F=12288, V=151936, mask_id=151935)
    w = B.Weights(w_qkv=0x1000, w_o=0x1000, w_gateup=0x1000, w_down=0x1000, g_attn=0x1000, g_ffn=0x1000,
                  g_final=0x1000, embed=0x1000, lm_head=0x1000)
    for Bn, g, fits in [(1, 16, True), (4, 16, True), (1, 33, False), (8, 16, False)]:
        c = _cache(Bn=Bn, cap=4096, lens=[2048] * Bn)
        with pytest.raises(B.DFlashError) as e:
            B.draft_forward_noalloc(_dims(**qwen), w, c, 0x4000, None, g, 0x5000)
        if fits:
            assert e.value.status != B.ERR_WORKSPACE, B.last_error()
        else:
            assert e.value.status == B.ERR_WORKSPACE and "no-allocation" in B.last_error()


def test_target_verify_checks(lib):
    w = B.Weights(w_qkv=0x1000, w_o=0x1000, w_gateup=0x1000, w_down=0x1000, g_attn=0x1000, g_ffn=0x1000,
                  g_final=0x1000, embed=0x1000, lm_head=0x1000)
    taps = [0x8000] * 5
    ok_layers = [0, 1, 2, 3, 4]

    def call(**kw):
        a = dict(dims=_dims(L=8), w=w, cache=_cache(lens=(10, 0)), tok=0x4000, gamma=16, layers=ok_layers, taps=taps,
                 out=0x5000, ws=0x100000, nbytes=1 << 30)
        a.update(kw)
        with pytest.raises(B.DFlashError) as e:
            B.target_verify(a["dims"], a["w"], a["cache"], a["tok"], a["gamma"], a["layers"], a["taps"], a["out"],
                            None, a["ws"], a["nbytes"])
        return e.value.status

    assert call(gamma=0) == B.ERR_INVALID_ARG
    assert call(gamma=34) == B.ERR_INVALID_ARG
    assert call(layers=[0, 1, 2, 3, 8]) == B.ERR_INVALID_ARG      # layer outside [0, L)
    assert call(layers=[0, 2, 1, 3, 4]) == B.ERR_INVALID_ARG      # not increasing
    assert call(taps=[0x8000] * 4 + [0x8001]) == B.ERR_INVALID_ARG   # misaligned tap buffer
    assert call(out=0) == B.ERR_INVALID_ARG
    assert call(cache=_cache(cap=64, lens=(50, 0))) == B.ERR_CAPACITY
    assert call(nbytes=16) == B.ERR_WORKSPACE
    # gamma 1 (a plain decoding step) passes the argument checks
    assert call(gamma=1) not in (B.ERR_INVALID_ARG, B.ERR_CAPACITY, B.ERR_WORKSPACE)


def test_workspace_covers_target_verify(lib):
    qwen = _dims(D=4096, L=36, Hq=32, Hkv=8, head_dim=128, F=12288, V=151936, mask_id=151935)
    assert B.workspace_size(qwen, 1, 16, 0) > 0


def test_len_dev_alignment(lib):
    with pytest.raises(B.DFlashError) as e:
        B.inject_kv(_dims(), B.Weights(w_qkv=0x1000), 0x3000, [1, 1], _cache(len_dev=0x3002), 0, 0)
    assert e.value.status == B.ERR_INVALID_ARG and "len_dev" in B.last_error()


def test_workspace_too_small(lib):
    w = B.Weights(w_qkv=0x1000, w_o=0x1000, w_gateup=0x1000, w_down=0x1000, g_attn=0x1000, g_ffn=0x1000,
                  g_final=0x1000, embed=0x1000, lm_head=0x1000)
    with pytest.raises(B.DFlashError) as e:
        B.draft_forward(_dims(), w, _cache(), 0x4000, None, 16, 0x5000, 0x100000, 16)
    assert e.value.status == B.ERR_WORKSPACE
    with pytest.raises(B.DFlashError) as e:
        B.draft_forward(_dims(), w, _cache(), 0x4000, None, 16, 0x5000, 0, 0)
    assert e.value.status == B.ERR_WORKSPACE


def test_misaligned_and_bad_cache(lib):
    w = B.Weights(w_c=0x1001, g_c=0x1000)
    with pytest.raises(B.DFlashError) as e:
        B.fuse_context(_dims(), w, [0x2000] * 5, 256, 4, 0x3000, 0x100000, 1 << 30)
    assert e.value.status == B.ERR_INVALID_ARG
    w = B.Weights(w_c=0x1000, g_c=0x1000)
    with pytest.raises(B.DFlashError) as e:     # ld < D
        B.fuse_context(_dims(), w, [0x2000] * 5, 128, 4, 0x3000, 0x100000, 1 << 30)
    assert e.value.status == B.ERR_INVALID_ARG
    with pytest.raises(B.DFlashError) as e:     # cap not a multiple of 32
        B.inject_kv(_dims(), B.Weights(w_qkv=0x1000), 0x3000, [1, 1], _cache(cap=60), 0, 0)
    assert e.value.status == B.ERR_INVALID_ARG
    with pytest.raises(B.DFlashError) as e:     # a multiple of 8 but not of 32
        B.inject_kv(_dims(), B.Weights(w_qkv=0x1000), 0x3000, [1, 1], _cache(cap=40), 0, 0)
    assert e.value.status == B.ERR_INVALID_ARG
    with pytest.raises(B.DFlashError) as e:     # B too large
        B.inject_kv(_dims(), B.Weights(w_qkv=0x1000), 0x3000, [1] * 65,
                    _cache(Bn=65, lens=[0] * 65), 0, 0)
    assert e.value.status == B.ERR_INVALID_ARG
    with pytest.raises(B.DFlashError) as e:     # negative rows
        B.inject_kv(_dims(), B.Weights(w_qkv=0x1000), 0x3000, [-1, 1], _cache(), 0, 0)
    assert e.value.status == B.ERR_INVALID_ARG


def test_argmax_accept_flags(lib):
    for flags in (0, 4, 7):
        with pytest.raises(B.DFlashError) as e:
            B.argmax_accept(_dims(), B.Weights(lm_head=0x1000), flags, 0x2000, 1, 16, 0x3000, 0x4000,
                            0x5000, 0x6000, None, None, 0, 0)
        assert e.value.status == B.ERR_INVALID_ARG
    with pytest.raises(B.DFlashError) as e:     # ACCEPT needs target/tau/next
        B.argmax_accept(_dims(), None, B.ACCEPT, None, 1, 16, 0x3000, None, 0x5000, 0x6000, None, None, 0, 0)
    assert e.value.status == B.ERR_INVALID_ARG


def test_empty_calls_are_noops(lib):
    # T = 0 and all-zero row counts return OK without touching the device
    B.fuse_context(_dims(), B.Weights(), [0] * 5, 256, 0, 0, 0, 0)
    c = _cache(lens=(3, 4))
    B.inject_kv(_dims(), B.Weights(), 0, [0, 0], c, 0, 0)
    assert list(c._keep) == [3, 4]


def test_workspace_covers_smaller_calls(lib):
    # the returned size bounds every call with fewer sequences / a shorter block
    d = _dims(D=1024, F=2048, Hq=8, Hkv=2, head_dim=128, V=5000, L=2)
    big = B.workspace_size(d, 4, 33, 3000)
    for b in (1, 2, 4):
        for g in (2, 8, 16, 17, 32, 33):
            assert B.workspace_size(d, b, g, 3000) <= big
    for rows in (1, 16, 100, 3000):
        assert B.workspace_size(d, 4, 33, rows) <= big


def test_profile_hook_validation(lib):
    assert B.profile_events(B.PROF_NONE) == 0
    with pytest.raises(B.DFlashError) as e:
        B.profile_events(42)
    assert e.value.status == B.ERR_INVALID_ARG


@pytest.mark.parametrize("T", [0.0, -1.0, float("nan"), float("inf"), 1e-45])
def test_sampling_temperature_rejected(lib, T):
    with pytest.raises(B.DFlashError) as e:
        B.sample_drafts(_dims(), B.Weights(lm_head=0x1000), 0x2000, 1, 16, T, 0x3000, 0x4000, 0x5000, None, 0, 0)
    assert e.value.status == B.ERR_INVALID_ARG and "temperature" in B.last_error()
    with pytest.raises(B.DFlashError) as e:
        B.sample_accept(_dims(), 1, 16, T, 0x1000, 0x2000, None, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000, 0, 0)
    assert e.value.status == B.ERR_INVALID_ARG


def test_sampling_arguments_checked(lib):
    W = B.Weights(lm_head=0x1000)
    good = dict(h=0x2000, u=0x3000, d=0x4000, z=0x5000)
    for miss in good:
        a = dict(good)
        a[miss] = None
        with pytest.raises(B.DFlashError) as e:
            B.sample_drafts(_dims(), W, a["h"], 1, 16, 1.0, a["u"], a["d"], a["z"], None, 0, 0)
        assert e.value.status == B.ERR_INVALID_ARG, miss
    with pytest.raises(B.DFlashError) as e:       # misaligned logits
        B.sample_drafts(_dims(), W, 0x2000, 1, 16, 1.0, 0x3000, 0x4000, 0x5004, None, 0, 0)
    assert e.value.status == B.ERR_INVALID_ARG
    with pytest.raises(B.DFlashError) as e:       # batch out of range
        B.sample_drafts(_dims(), W, 0x2000, 65, 16, 1.0, 0x3000, 0x4000, 0x5000, None, 0, 0)
    assert e.value.status == B.ERR_INVALID_ARG
    with pytest.raises(B.DFlashError) as e:       # no workspace
        B.sample_drafts(_dims(), W, 0x2000, 1, 16, 1.0, 0x3000, 0x4000, 0x5000, None, 0, 0)
    assert e.value.status == B.ERR_WORKSPACE
    acc = dict(d=0x1000, z=0x2000, t=0x3000, au=0x4000, ru=0x5000, tau=0x6000, nxt=0x7000)
    for miss in acc:
        a = dict(acc)
        a[miss] = None
        with pytest.raises(B.DFlashError) as e:
            B.sample_accept(_dims(), 1, 16, 1.0, a["d"], a["z"], None, a["t"], a["au"], a["ru"], a["tau"],
                            a["nxt"], 0, 0)
        assert e.value.status == B.ERR_INVALID_ARG, miss
    with pytest.raises(B.DFlashError) as e:       # gamma out of range
        B.sample_accept(_dims(), 1, 34, 1.0, 0x1000, 0x2000, None, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000, 0, 0)
    assert e.value.status == B.ERR_INVALID_ARG
    with pytest.raises(B.DFlashError) as e:       # workspace too small
        B.sample_accept(_dims(), 1, 16, 1.0, 0x1000, 0x2000, None, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000,
                        0x10000, 16)
    assert e.value.status == B.ERR_WORKSPACE


def test_ragged_draft_checks(lib):
    w = B.Weights(w_qkv=0x1000, w_o=0x1000, w_gateup=0x1000, w_down=0x1000, g_attn=0x1000, g_ffn=0x1000,
                  g_final=0x1000, embed=0x1000, lm_head=0x1000)
    for gammas in ([16, 1], [34, 16], [0, 2]):           # a block length outside [2, 33]
        with pytest.raises(B.DFlashError) as e:
            B.draft_forward_ragged(_dims(), w, _cache(), 0x4000, None, gammas, 0x5000, 0x100000, 1 << 30)
        assert e.value.status == B.ERR_INVALID_ARG
    c = _cache(lens=(10, 40))
    with pytest.raises(B.DFlashError) as e:              # only the second sequence overflows: 40 + 30 > 64
        B.draft_forward_ragged(_dims(), w, c, 0x4000, None, [33, 30], 0x5000, 0x100000, 1 << 30)
    assert e.value.status == B.ERR_CAPACITY and "sequence 1" in B.last_error()
    assert list(c._keep) == [10, 40]
    with pytest.raises(B.DFlashError) as e:              # workspace sized for a shorter block
        small_ws = B.workspace_size(_dims(), 2, 4, 1)
        B.draft_forward_ragged(_dims(), w, _cache(), 0x4000, None, [4, 20], 0x5000, 0x100000, small_ws)
    assert e.value.status == B.ERR_WORKSPACE


def test_ragged_argmax_accept_checks(lib):
    W = B.Weights(lm_head=0x1000)
    with pytest.raises(B.DFlashError) as e:
        B.argmax_accept_ragged(_dims(), W, B.ARGMAX, 0x2000, [16, 1], 0x3000, None, None, None, None, None,
                               0x100000, 1 << 30)
    assert e.value.status == B.ERR_INVALID_ARG
    with pytest.raises(B.DFlashError) as e:              # ACCEPT needs target / tau / next
        B.argmax_accept_ragged(_dims(), None, B.ACCEPT, None, [4, 8], 0x3000, None, 0x5000, 0x6000, None, None,
                               0, 0)
    assert e.value.status == B.ERR_INVALID_ARG
    with pytest.raises(B.DFlashError) as e:
        B.argmax_accept_ragged(_dims(), W, B.ARGMAX, 0x2000, [4, 8], 0x3000, None, None, None, None, None, 0, 0)
    assert e.value.status == B.ERR_WORKSPACE


def test_workspace_covers_ragged_row_counts(lib):
    # every total row count a ragged call can reach is covered by the size for
    # its longest block (prime totals included)
    d = _dims(D=1024, F=2048, Hq=8, Hkv=2, head_dim=128, V=5000, L=2)
    big = B.workspace_size(d, 4, 16, 1)
    assert big >= B.workspace_size(d, 4, 15, 1)
    assert big >= B.workspace_size(d, 3, 16, 1)


def test_blocks_checks(lib, monkeypatch):
    w = B.Weights(w_qkv=0x1000, w_o=0x1000, w_gateup=0x1000, w_down=0x1000, g_attn=0x1000, g_ffn=0x1000,
                  g_final=0x1000, embed=0x1000, lm_head=0x1000)
    c = _cache(cap=128, lens=(40, 10))
    for seqs, anchors in (([2], [0]), ([0], [41]), ([1], [-1]), ([0] * 65, [0] * 65)):
        with pytest.raises(B.DFlashError) as e:
            B.draft_forward_blocks(_dims(), w, c, seqs, anchors, 16, 0x4000, None, 0x5000, 0x100000, 1 << 30)
        assert e.value.status == B.ERR_INVALID_ARG, (seqs, anchors)
    # sequence 0: context rounds up to 64; its blocks 0, 2, 4 are not
    # consecutive, so three 32-row slots reach 160 > 128
    with pytest.raises(B.DFlashError) as e:
        B.draft_forward_blocks(_dims(), w, c, [0, 1, 0, 1, 0], [5, 3, 40, 0, 0], 16, 0x4000, None, 0x5000,
                               0x100000, 1 << 30)
    assert e.value.status == B.ERR_CAPACITY and "block 4" in B.last_error()
    assert list(c._keep) == [40, 10]
    # four consecutive blocks of sequence 0 form two pairs (bf16 weights, fp32
    # cache), one 32-row slot each: rows [64, 128) fit, and the call gets as
    # far as the device check; one block per group they would need 192 rows
    with pytest.raises(B.DFlashError) as e:
        B.draft_forward_blocks(_dims(), w, c, [0, 0, 0, 0], [5, 40, 3, 0], 16, 0x4000, None, 0x5000, 0x100000,
                               1 << 30)
    assert e.value.status == B.ERR_HIP
    monkeypatch.setenv("DFLASH_BLOCK_PAIRS", "2")
    with pytest.raises(B.DFlashError) as e:
        B.draft_forward_blocks(_dims(), w, c, [0, 0, 0, 0], [5, 40, 3, 0], 16, 0x4000, None, 0x5000, 0x100000,
                               1 << 30)
    assert e.value.status == B.ERR_CAPACITY and "block 2" in B.last_error()
    monkeypatch.delenv("DFLASH_BLOCK_PAIRS")
    with pytest.raises(B.DFlashError) as e:
        B.draft_forward_blocks(_dims(), w, c, [0, 1], [5, 3], 16, 0x4000, None, 0x5000, 0x100000, 16)
    assert e.value.status == B.ERR_WORKSPACE
