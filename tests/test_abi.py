"""C-ABI library checks that need no GPU.

The library loads and exports every function include/moe_slot.h declares;
slab layouts agree with the generator and the oracle; argument errors come
back as status codes with a reason (no GPU call is made on those paths); and
the CPU host pass (moe_ffn_host_misses) matches the oracle's host share.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def mlib():
    from expert_vram_slot_amd import build as b
    if not os.path.exists(b.LIB):
        b.build()
    import expert_vram_slot_amd as m
    m.lib()
    return m


def test_exports_every_declared_function(mlib):
    from expert_vram_slot_amd import build as b
    api = b.exported_api()
    assert set(api) >= {"moe_route", "cache_manage", "cache_gather", "moe_ffn_slots", "moe_ffn_host_misses",
                        "moe_combine", "moe_bias_table", "cache_init", "cache_pick_static", "moe_slab_layout",
                        "moe_ffn_workspace_bytes", "moe_host_alloc", "moe_host_free", "moe_abi_version",
                        "moe_last_error"}
    out = subprocess.run(["nm", "-D", "--defined-only", b.LIB], capture_output=True, text=True, check=True).stdout
    have = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    assert not [n for n in api if n not in have]
    L = ctypes.CDLL(b.LIB)
    for n in api:
        assert getattr(L, n) is not None


def test_version(mlib):
    assert mlib.moe_abi_version() == 1


@pytest.mark.parametrize("w_type,H,I", [(0, 64, 128), (1, 2048, 768), (2, 2048, 768), (3, 2048, 512),
                                        (1, 4096, 1536)])
def test_slab_layout_matches_generator_and_oracle(mlib, w_type, H, I):
    lay = mlib.moe_slab_layout(w_type, H, I)
    assert lay.total == synth.slab_bytes(w_type, H, I) == oracle.slab_bytes(w_type, H, I)
    for p in range(3):
        assert lay.w[p] % 16 == 0
        if lay.s[p] >= 0:
            assert lay.s[p] % 16 == 0


def test_slab_layout_planes_hold_the_encoded_matrices(mlib):
    """Offsets of the layout point at the generator's planes (fp32 / int8)."""
    H, I = 64, 32
    rng = np.random.default_rng(0)
    wg, wu = rng.normal(0, 1, (I, H)).astype(np.float32), rng.normal(0, 1, (I, H)).astype(np.float32)
    wd = rng.normal(0, 1, (H, I)).astype(np.float32)
    slab = synth.encode_slab(0, H, I, wg, wu, wd)
    lay = mlib.moe_slab_layout(0, H, I)
    for p, m in enumerate((wg, wu, wd)):
        got = slab[lay.w[p]:lay.w[p] + m.nbytes].view(np.float32).reshape(m.shape)
        np.testing.assert_array_equal(got, m)
    slab8 = synth.encode_slab(2, H, I, wg, wu, wd)
    lay8 = mlib.moe_slab_layout(2, H, I)
    sd = slab8[lay8.s[2]:lay8.s[2] + 4 * H].view(np.float32)
    np.testing.assert_allclose(sd, np.abs(wd).max(axis=1) / 127, rtol=1e-6)


def test_layout_refusals(mlib):
    with pytest.raises(mlib.MoeError) as e:
        mlib.moe_slab_layout(3, 2048, 520)
    assert e.value.code == mlib.MOE_E_ALIGN and "multiples of 32" in str(e.value)
    with pytest.raises(mlib.MoeError) as e:
        mlib.moe_slab_layout(9, 64, 64)
    assert e.value.code == mlib.MOE_E_DTYPE


def test_argument_errors_return_codes_without_gpu_work(mlib):
    L = mlib.lib()
    # NULL inputs
    assert L.moe_route(None, 1, None, None, None, 4, 64, 8, 2, None, None, None, None) == mlib.MOE_E_ARG
    assert "non-NULL" in mlib.moe_last_error()
    # k > E
    assert L.moe_route(16, 1, 16, None, None, 4, 64, 8, 9, 16, 16, None, None) == mlib.MOE_E_SHAPE
    # wrong activation format for the weight format
    assert L.moe_ffn_slots(16, 0, 16, 16, 4, 2, 16, 6 * 64 * 128, 4, 1, 64, 128, 16, 16, 1 << 20,
                           None) == mlib.MOE_E_DTYPE
    # slab not a 16-byte multiple / too small
    assert L.moe_ffn_slots(16, 1, 16, 16, 4, 2, 16, 1000, 4, 1, 64, 128, 16, 16, 1 << 20, None) == mlib.MOE_E_ALIGN
    # misaligned store pointer
    assert L.cache_gather(16, 16, 4, 24, 32, 96, None) == mlib.MOE_E_ALIGN
    # workspace too small
    assert L.moe_ffn_slots(16, 1, 16, 16, 4, 2, 16, 6 * 64 * 128, 4, 1, 64, 128, 16, 16, 64, None) == mlib.MOE_E_ARG
    # cache state: S > E
    st = mlib.CacheState(16, 16, 16, 16, 16, 4, 8)
    assert L.cache_manage(ctypes.byref(st), 1, 16, 8, 16, 16, 16, 16, 16, None, None) == mlib.MOE_E_SHAPE
    # unknown policy
    st = mlib.CacheState(16, 16, 16, 16, 16, 8, 4)
    assert L.cache_manage(ctypes.byref(st), 7, 16, 8, 16, 16, 16, 16, 16, None, None) == mlib.MOE_E_ARG
    # bias cap must be <= 0
    assert L.moe_bias_table(16, 8, 2, ctypes.c_float(0.5), 16, None) == mlib.MOE_E_ARG


def test_workspace_bytes_grow_with_batch(mlib):
    a = mlib.moe_ffn_workspace_bytes(1, 8, 64, 1, 2048, 768)
    b = mlib.moe_ffn_workspace_bytes(64, 8, 64, 1, 2048, 768)
    assert 0 < a < b
    assert b >= 64 * 8 * 2048 * 4  # per-pick partial outputs
    assert mlib.moe_ffn_workspace_bytes(4, 0, 4, 1, 64, 64) == 0


# ------------------------------------------------------------ host pass


def _host_case(cfg, T, S, n_threads, E=None, seed_step=0):
    li = synth.LayerInputs(cfg, T=T, step=seed_step, E=E)
    z = oracle.logits(li.x, li.x_dtype, li.G)
    ids = oracle.topk(z, li.k)
    w = oracle.route_weights(z, ids)
    resident = list(range(0, 2 * S, 2))[:S]
    c = oracle.Cache(li.E, S, "static", resident=resident)
    sl = c.manage(ids)["slot_ids"].reshape(ids.shape)
    _, yg, yh = oracle.layer(li.w_type, li.store, li.E, li.H, li.I, li.x, li.x_dtype, ids, w, sl)
    return li, ids, w, sl, yg, yh


def _run_host(mlib, li, ids, w, sl, n_threads):
    y = np.full((li.T, li.H), np.nan, np.float32)
    mlib.moe_ffn_host_misses(li.x, li.x_dtype, ids, sl, w, li.T, li.k, li.store, li.slab, li.E, li.w_type, li.H,
                             li.I, y, n_threads)
    return y


TOL = {0: (1e-5, None), 1: (2e-2, 1e-2), 2: (3e-2, None), 3: (3e-2, None)}


def _assert_close(got, ref, w_type):
    rtol, atol = TOL[w_type]
    rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2))) or 1.0
    if atol is None:
        atol = rtol * rms
    err = np.abs(got.astype(np.float64) - ref) - (rtol * np.abs(ref) + atol)
    assert np.all(err <= 0), f"max excess {err.max():.3e} (rms {rms:.3e})"


@pytest.mark.parametrize("cfg,T,S,E", [("c1", 16, 4, None), ("c2", 4, 64, None), ("c3", 3, 32, None),
                                       ("c4", 2, 192, None)])
def test_host_pass_matches_oracle_host_share(mlib, cfg, T, S, E):
    li, ids, w, sl, yg, yh = _host_case(cfg, T, S, 4, E=E)
    y = _run_host(mlib, li, ids, w, sl, 4)
    _assert_close(y, yh, li.w_type)
    # tokens whose every pick is resident get exactly +0.0
    full = np.all(sl >= 0, axis=1)
    assert np.all(y[full] == 0) and not np.any(np.signbit(y[full]))


def test_host_pass_thread_count_does_not_change_bits(mlib):
    li, ids, w, sl, yg, yh = _host_case("c2", 4, 32, 1)
    a = _run_host(mlib, li, ids, w, sl, 1)
    b = _run_host(mlib, li, ids, w, sl, 7)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("cfg,T,S,E", [("c4", 12, 8, 32), ("c2", 16, 4, 16), ("c3", 16, 4, 16)])
def test_host_pass_many_picks_per_expert(mlib, cfg, T, S, E):
    # most experts carry several picks, so each weight row is read (and for
    # 4-bit decoded) once for groups of up to four picks, and more than four
    # spill into a second group; bits must not depend on the thread count
    li, ids, w, sl, yg, yh = _host_case(cfg, T, S, 4, E=E)
    counts = np.bincount(ids[sl < 0], minlength=E)
    assert counts.max() > 4
    a = _run_host(mlib, li, ids, w, sl, 1)
    _assert_close(a, yh, li.w_type)
    np.testing.assert_array_equal(a, _run_host(mlib, li, ids, w, sl, 5))


def test_host_pass_q4_rows_not_in_whole_groups(mlib):
    # H = 96, I = 160: 32-weight blocks but not whole groups of four blocks
    E, k, H, I, T = 6, 2, 96, 160, 5
    base = synth.config_seed("c4")
    x = synth.normal(synth.key(base, synth.TAG_X, 3, 0), (T, H), 1.0, synth.X_BF16)
    G = synth.normal(synth.key(base, synth.TAG_G, 3, 0), (E, H), 0.5, synth.X_BF16)
    store = synth.slabs(synth.W_Q4B32, base, 3, 0, E, H, I, 0.05)
    z = oracle.logits(x, synth.X_BF16, G)
    ids = oracle.topk(z, k)
    w = oracle.route_weights(z, ids)
    sl = np.where(ids % 2 == 0, -1, 0).astype(np.int32)
    _, _, yh = oracle.layer(synth.W_Q4B32, store, E, H, I, x, synth.X_BF16, ids, w, sl)
    y = np.full((T, H), np.nan, np.float32)
    mlib.moe_ffn_host_misses(x, synth.X_BF16, ids, sl, w, T, k, store, synth.slab_bytes(synth.W_Q4B32, H, I), E,
                             synth.W_Q4B32, H, I, y, 3)
    _assert_close(y, yh, synth.W_Q4B32)


@pytest.mark.parametrize("w_type,H,I", [(synth.W_W8A8, 96, 160), (synth.W_W8A8, 80, 112), (synth.W_W8A8, 128, 192),
                                         (synth.W_BF16, 80, 112), (synth.W_BF16, 96, 160)])
def test_host_pass_row_lengths_of_every_dot_path(mlib, w_type, H, I):
    # the host pass picks its dot products by row length: W8A8 rows in whole
    # 64s take the VNNI path (128 / 192), in 32s the int16 path (96 / 160),
    # others the scalar one (80 / 112); bf16 rows in 32s the AVX-512 BF16 path,
    # others the scalar one.  Each against the oracle, several picks per
    # expert so the grouped row passes run, bits independent of the threads.
    E, k, T = 6, 3, 9
    base = synth.config_seed("c3")
    x = synth.normal(synth.key(base, synth.TAG_X, 5, H), (T, H), 1.0, synth.X_BF16)
    G = synth.normal(synth.key(base, synth.TAG_G, 5, H), (E, H), 0.5, synth.X_BF16)
    store = synth.slabs(w_type, base, 5, 0, E, H, I, 0.05)
    z = oracle.logits(x, synth.X_BF16, G)
    ids = oracle.topk(z, k)
    w = oracle.route_weights(z, ids)
    sl = np.where(ids % 3 == 0, 0, -1).astype(np.int32)
    _, _, yh = oracle.layer(w_type, store, E, H, I, x, synth.X_BF16, ids, w, sl)
    slab = synth.slab_bytes(w_type, H, I)
    ys = []
    for nt in (1, 4):
        y = np.full((T, H), np.nan, np.float32)
        mlib.moe_ffn_host_misses(x, synth.X_BF16, ids, sl, w, T, k, store, slab, E, w_type, H, I, y, nt)
        ys.append(y)
    _assert_close(ys[0], yh, w_type)
    np.testing.assert_array_equal(ys[0], ys[1])


def test_host_pass_all_miss_is_the_whole_layer(mlib):
    li = synth.LayerInputs("c1")
    z = oracle.logits(li.x, 0, li.G)
    ids = oracle.topk(z, 2)
    w = oracle.route_weights(z, ids)
    yf, _, _ = oracle.layer(0, li.store, 8, 64, 128, li.x, 0, ids, w)
    y = _run_host(mlib, li, ids, w, np.full_like(ids, -1), 3)
    _assert_close(y, yf, 0)


def test_host_pass_scratch_kept_between_calls(mlib):
    # the pass keeps its intermediate rows between calls on one thread: a
    # call after larger ones, in other formats and with other residency, must
    # give the bits it gives first, and a token with no host pick exactly +0.0
    li, ids, w, sl, yg, yh = _host_case("c2", 4, 32, 1)
    first = _run_host(mlib, li, ids, w, sl, 3)
    for cfg, T, S in (("c2", 12, 16), ("c3", 8, 8), ("c4", 6, 96), ("c1", 16, 4)):
        o = _host_case(cfg, T, S, 3)
        _run_host(mlib, o[0], o[1], o[2], o[3], 3)
    np.testing.assert_array_equal(_run_host(mlib, li, ids, w, sl, 3), first)
    # now every pick of token 0 resident: its row must not pick up rows left
    # by the calls before
    sl2 = sl.copy()
    sl2[0] = np.maximum(sl2[0], 0)
    y2 = _run_host(mlib, li, ids, w, sl2, 3)
    assert np.all(y2[0] == 0) and not np.any(np.signbit(y2[0]))
    np.testing.assert_array_equal(y2[1:], first[1:])
