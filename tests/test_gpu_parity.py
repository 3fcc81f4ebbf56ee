"""GPU parity: every entry point of libmoeslot.so against the CPU oracle.

Bars: routing ids, slot maps, miss and host lists, cache state and gathered
bytes bit-exact; outputs within |d| <= rtol*|ref| + atol, with (rtol, atol)
= (1e-5, 1e-5*rms) for fp32, (2e-2, 1e-2) for bf16 and (3e-2, 3e-2*rms) for
int8 and 4-bit weights.
"""
import functools

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def m():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import expert_vram_slot_amd as mod
    mod.lib()
    return mod


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


TOL = {0: (1e-5, None), 1: (2e-2, 1e-2), 2: (3e-2, None), 3: (3e-2, None)}


def assert_close(got, ref, w_type, what=""):
    rtol, atol = TOL[w_type]
    ref = ref.astype(np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2))) or 1.0
    if atol is None:
        atol = rtol * rms
    excess = np.abs(got.astype(np.float64) - ref) - (rtol * np.abs(ref) + atol)
    assert np.all(excess <= 0), f"{what}: max excess {excess.max():.3e} at {np.unravel_index(excess.argmax(), excess.shape)} (rms {rms:.3e})"


def x_torch_dtype(x_dtype):
    return torch.float32 if x_dtype == 0 else torch.int16


# ------------------------------------------------------------------ router


def gpu_route(m, li, bias=None, ids_in=None, with_logits=True):
    """moe_route on the GPU; with a logits buffer it runs as logits + top-k
    kernels, without one as the fused per-token-block kernel (z is None)."""
    T, H, E, k = li.T, li.H, li.E, li.k
    x = dev(li.x.view(np.int16) if li.x_dtype else li.x)
    G = dev(li.G.view(np.int16) if li.x_dtype else li.G)
    ids = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    z = torch.empty((T, E), dtype=torch.float32, device="cuda") if with_logits else None
    b = None if bias is None else dev(bias)
    ii = None if ids_in is None else dev(ids_in)
    m.moe_route(x, li.x_dtype, G, b, ii, T, H, E, k, ids, w, z)
    return host(ids), host(w), None if z is None else host(z)


def check_route(m, li, bias=None):
    ids, w, z = gpu_route(m, li, bias)
    zo = oracle.logits(li.x, li.x_dtype, li.G)
    # logits: one rounding of a double sum on both sides
    ulp = np.spacing(np.abs(zo))
    assert np.all(np.abs(z - zo) <= ulp)
    assert np.mean(z == zo) > 0.999
    # picks on the GPU's own logits: bit-exact
    np.testing.assert_array_equal(ids, oracle.topk(z, li.k, bias))
    # end-to-end picks at this seed: bit-exact
    np.testing.assert_array_equal(ids, oracle.topk(zo, li.k, bias))
    np.testing.assert_allclose(w, oracle.route_weights(z, ids), rtol=2e-6, atol=1e-9)
    return ids, w, z


@pytest.mark.parametrize("cfg,T", [("c1", 16), ("c2", 1), ("c2", 8), ("c2", 64), ("c3", 16), ("c4", 1),
                                   ("c4", 32), ("c2", 300)])
def test_route_matches_oracle(m, cfg, T):
    li = synth.LayerInputs(cfg, T=T, with_store=False)
    check_route(m, li)


@pytest.mark.parametrize("cfg,T", [("c1", 16), ("c2", 1), ("c2", 64), ("c4", 32), ("c2", 300)])
def test_route_fused_kernel_matches_oracle(m, cfg, T):
    """Without a logits buffer the router runs as one fused kernel per token block."""
    li = synth.LayerInputs(cfg, T=T, with_store=False)
    ids, w, _ = gpu_route(m, li, with_logits=False)
    zo = oracle.logits(li.x, li.x_dtype, li.G)
    np.testing.assert_array_equal(ids, oracle.topk(zo, li.k))
    np.testing.assert_allclose(w, oracle.route_weights(zo, ids), rtol=4e-6, atol=1e-9)
    ids2, w2, z2 = gpu_route(m, li)
    np.testing.assert_array_equal(ids2, ids)
    np.testing.assert_allclose(w2, w, rtol=4e-6, atol=1e-9)


def test_route_prefill_shape(m):
    li = synth.LayerInputs("c5", T=2048, with_store=False)
    check_route(m, li)


@pytest.mark.parametrize("T,E,H,k", [(517, 77, 96, 4), (600, 40, 32, 8), (512, 288, 4096, 8)])
def test_route_matrix_core_logits_ragged(m, T, E, H, k):
    """bf16 batches of 512 tokens and more take the fp64 matrix-core logits:
    token and expert counts off the 16 / 32 tiles (a partial and an empty
    expert tile), h of three 32-input blocks (halves of two and one) and of
    one block (one wave pair with nothing to add), and the 288-expert gate."""
    x = synth.normal(synth.key(T, 31, E), (T, H), 1.0, 1)
    G = synth.normal(synth.key(T, 32, H), (E, H), 0.05, 1)
    li = type("L", (), dict(T=T, H=H, E=E, k=k, x=x, x_dtype=1, G=G))
    check_route(m, li)


def test_route_with_graded_bias(m):
    li = synth.LayerInputs("c4", T=32, with_store=False, layer=3)
    b = synth.dirichlet(synth.key(li.base, synth.TAG_B, 3), li.E, 0.3)
    bias_o = oracle.bias_table(b, 192, -1.0)
    bias_g = torch.empty(li.E, dtype=torch.float32, device="cuda")
    m.moe_bias_table(dev(b), li.E, 192, -1.0, bias_g)
    bias_g = host(bias_g)
    assert np.all(np.abs(bias_g - bias_o) <= np.spacing(np.abs(bias_o)))
    np.testing.assert_array_equal(bias_g == 0, bias_o == 0)
    ids, w, z = check_route(m, li, bias_o)
    # the bias moved some picks, and the weights stayed the raw-logit softmax
    assert np.any(ids != oracle.topk(z, li.k))


@pytest.mark.parametrize("value", [-0.75, -np.inf])
def test_flat_bias_and_hard_mask_match_oracle(m, value):
    """Flat soft bias and hard mask tables, and the routing under them."""
    li = synth.LayerInputs("c4", T=32, with_store=False, layer=5)
    b = synth.dirichlet(synth.key(li.base, synth.TAG_B, 5), li.E, 0.3)
    bias_o = oracle.bias_flat(b, 192, value)
    bias_g = torch.empty(li.E, dtype=torch.float32, device="cuda")
    m.moe_bias_flat(dev(b), li.E, 192, value, bias_g)
    np.testing.assert_array_equal(host(bias_g), bias_o)
    ids, w, z = check_route(m, li, bias_o)
    if value == -np.inf:
        assert np.all(bias_o[ids] == 0.0)  # only hot experts are picked


def test_affinity_bias_follows_the_live_cache(m):
    """The affinity table is read from the cache state on the device: after a
    manage step it adds lambda exactly to the experts that now have a slot."""
    E, S, k, T = 128, 32, 8, 16
    li = synth.LayerInputs("c2", T=T, with_store=False, layer=2)
    c = GpuCache(m, E, S)
    ids0 = synth.zipf_ids(synth.key(li.base, synth.TAG_ZIPF_PERM, 2), synth.key(li.base, synth.TAG_ZIPF_DRAW, 2), T, E,
                          k, 0.8)
    c.manage("lru", ids0)
    e2s = host(c.e2s)
    base_o = oracle.bias_flat(synth.dirichlet(synth.key(li.base, synth.TAG_B, 2), E, 0.3), 48, -0.5)
    for base in (None, base_o):
        aff_o = oracle.bias_affinity(e2s, 0.25, base)
        aff_g = torch.empty(E, dtype=torch.float32, device="cuda")
        m.moe_bias_affinity(c.e2s, None if base is None else dev(base), E, 0.25, aff_g)
        np.testing.assert_array_equal(host(aff_g), aff_o)
        ids, w, z = check_route(m, li, aff_o)
    assert (e2s >= 0).sum() > 0


def test_route_damped_weights_match_oracle(m):
    li = synth.LayerInputs("c4", T=32, with_store=False, layer=6)
    b = synth.dirichlet(synth.key(li.base, synth.TAG_B, 6), li.E, 0.3)
    bias = oracle.bias_table(b, 192, -1.0)
    x = dev(li.x.view(np.int16)); G = dev(li.G.view(np.int16))
    for with_logits in (True, False):
        ids = torch.empty((li.T, li.k), dtype=torch.int32, device="cuda")
        w = torch.empty((li.T, li.k), dtype=torch.float32, device="cuda")
        z = torch.empty((li.T, li.E), dtype=torch.float32, device="cuda") if with_logits else None
        m.moe_route_ex(x, li.x_dtype, G, dev(bias), None, li.T, li.H, li.E, li.k, m.MOE_ROUTE_DAMPED, ids, w, z)
        zo = oracle.logits(li.x, li.x_dtype, li.G)
        ids_o = oracle.topk(zo, li.k, bias)
        np.testing.assert_array_equal(host(ids), ids_o)
        np.testing.assert_allclose(host(w), oracle.route_weights_damped(zo, bias, ids_o), rtol=4e-6, atol=1e-9)
    # flags 0 is moe_route; an unknown flag is refused
    with pytest.raises(m.MoeError):
        m.moe_route_ex(x, li.x_dtype, G, dev(bias), None, li.T, li.H, li.E, li.k, 2, ids, w, None)


def test_route_given_ids_only_weights(m):
    li = synth.LayerInputs("c3", T=16, with_store=False)
    ids_in = synth.zipf_ids(synth.key(li.base, synth.TAG_ZIPF_PERM), synth.key(li.base, synth.TAG_ZIPF_DRAW), 16,
                            li.E, li.k, 0.8)
    ids, w, z = gpu_route(m, li, ids_in=ids_in)
    np.testing.assert_allclose(w, oracle.route_weights(z, ids_in), rtol=2e-6, atol=1e-9)


def test_route_ties_go_to_lower_id(m):
    # integer-valued logits with many ties: G picks one column pattern
    T, H, E, k = 8, 16, 64, 6
    x = np.ones((T, H), np.float32)
    G = np.zeros((E, H), np.float32)
    G[:, 0] = np.arange(E) % 5  # five distinct logit values, many ties
    li = type("L", (), dict(T=T, H=H, E=E, k=k, x=x, G=G, x_dtype=0))
    ids, w, z = gpu_route(m, li)
    np.testing.assert_array_equal(ids, oracle.topk(z, k))
    assert list(ids[0]) == [4, 9, 14, 19, 24, 29]


# ------------------------------------------------------------------ cache


class GpuCache:
    def __init__(self, m, E, S, resident=None):
        self.m, self.E, self.S = m, E, S
        i32 = dict(dtype=torch.int32, device="cuda")
        self.e2s = torch.empty(E, **i32)
        self.s2e = torch.empty(max(S, 1), **i32)
        self.last = torch.empty(max(S, 1), **i32)
        self.freq = torch.empty(max(S, 1), **i32)
        self.step = torch.empty(1, **i32)
        self.st = m.cache_state(self.e2s, self.s2e, self.last, self.freq, self.step, E, S)
        m.cache_init(self.st, None if resident is None else dev(np.asarray(resident, np.int32)))
        self.miss = torch.empty(2 * max(S, 1), **i32)
        self.n_miss = torch.empty(1, **i32)
        self.host_miss = torch.empty(E, **i32)
        self.n_host = torch.empty(1, **i32)
        self.stats = torch.empty(4, **i32)

    def manage(self, policy, ids):
        ids = dev(np.asarray(ids, np.int32).reshape(-1))
        n = ids.numel()
        slot_ids = torch.full((max(n, 1),), -9, dtype=torch.int32, device="cuda")
        self.m.cache_manage(self.st, oracle.POLICIES[policy], ids, n, slot_ids, self.miss, self.n_miss,
                            self.host_miss, self.n_host, self.stats)
        nm, nh = int(host(self.n_miss)[0]), int(host(self.n_host)[0])
        return dict(slot_ids=host(slot_ids)[:n], miss=host(self.miss)[:2 * nm].reshape(nm, 2),
                    host_miss=host(self.host_miss)[:nh], stats=host(self.stats))


def phase_trace(base, n_tok, E, k, phase_len, s=0.8):
    """Routing ids whose popular handful changes: Zipf(s) over a permutation
    drawn anew for every phase of phase_len tokens."""
    out = []
    for ph in range((n_tok + phase_len - 1) // phase_len):
        n = min(phase_len, n_tok - ph * phase_len)
        out.append(synth.zipf_ids(synth.key(base, synth.TAG_ZIPF_PERM, 0, ph), synth.key(base, synth.TAG_ZIPF_DRAW, 0, ph),
                                  n, E, k, s))
    return np.concatenate(out)


@pytest.mark.parametrize("policy", ["static", "lru", "lfu", "repick"])
def test_policy_replay_matches_oracle(m, policy):
    """Replay of a routing trace one token per step: static set from the
    first window, LRU, LFU, and a static set repicked every `every` tokens
    from the last window's picks (cache_pick_static -> cache_repick ->
    cache_gather); stats, loads, state and slot contents equal the oracle's."""
    E, S, k, n_tok, every = 64, 16, 4, 600, 100
    trace = phase_trace(0xE55100AA, n_tok, E, k, 128)
    slab = 64
    store_h = np.arange(E * slab, dtype=np.uint32).astype(np.uint8).reshape(E, slab)
    store = torch.from_numpy(store_h.copy()).pin_memory()
    slots = torch.zeros((S, slab), dtype=torch.uint8, device="cuda")
    first = oracle.pick_static(trace[:every], E, S)
    pol = "static" if policy == "repick" else policy
    res = first if pol == "static" else None
    g = GpuCache(m, E, S, res)
    o = oracle.Cache(E, S, pol, res)
    if res is not None:
        slots.copy_(torch.from_numpy(store_h[first]).cuda())
    want = torch.empty(S, dtype=torch.int32, device="cuda")
    acc_g = np.zeros(4, np.int64)
    acc_o = np.zeros(4, np.int64)
    loads_g = loads_o = 0
    for t in range(n_tok):
        if policy == "repick" and t > 0 and t % every == 0:
            win = trace[t - every:t]
            m.cache_pick_static(dev(win.reshape(-1)), every * k, E, S, want)
            np.testing.assert_array_equal(host(want), oracle.pick_static(win, E, S))
            m.cache_repick(g.st, want, g.miss, g.n_miss)
            m.cache_gather(g.miss, g.n_miss, S, store, slots, slab)
            ld = o.repick(oracle.pick_static(win, E, S))
            nm = int(host(g.n_miss)[0])
            np.testing.assert_array_equal(host(g.miss)[:2 * nm].reshape(-1, 2), ld)
            loads_g += nm
            loads_o += len(ld)
        rg = g.manage(pol, trace[t])
        ro = o.manage(trace[t])
        if pol != "static":
            m.cache_gather(g.miss, g.n_miss, S, store, slots, slab)
        acc_g += rg["stats"]
        acc_o += ro["stats"]
    compare_state(g, o)
    np.testing.assert_array_equal(acc_g, acc_o)
    assert loads_g == loads_o
    # every occupied slot holds its expert's bytes
    s2e = host(g.s2e)[:S]
    for s_, e in enumerate(s2e):
        if e >= 0:
            np.testing.assert_array_equal(host(slots[s_]), store_h[e])
    if policy == "repick":
        assert loads_g > 0


@pytest.mark.parametrize("policy,E,S,T,k", [("lru", 64, 16, 4, 4), ("lfu", 64, 16, 4, 4), ("static", 64, 16, 4, 4),
                                             ("lru", 128, 32, 16, 8)])
def test_fused_manage_gather_and_doorbell(m, policy, E, S, T, k):
    """cache_manage_gather: the same state, lists and slot bytes as the
    oracle's manage + gather, step after step; the doorbell and the mirrored
    picks in pinned host memory match once seq has been written."""
    slab = 256
    store_h = (np.arange(E * slab, dtype=np.int64) * 7 % 251).astype(np.uint8).reshape(E, slab)
    store = torch.from_numpy(store_h.copy()).pin_memory()
    slots = torch.zeros((S, slab), dtype=torch.uint8, device="cuda")
    res = list(range(0, 2 * S, 2))[:S] if policy == "static" else None
    g = GpuCache(m, E, S, res)
    o = oracle.Cache(E, S, policy, res)
    if res is not None:
        slots.copy_(torch.from_numpy(store_h[res]).cuda())
    sync = torch.zeros(2, dtype=torch.int32, device="cuda")
    bell = torch.zeros(8, dtype=torch.int32).pin_memory()
    P = T * k
    b_ids = torch.full((P,), -5, dtype=torch.int32).pin_memory()
    b_slots = torch.full((P,), -5, dtype=torch.int32).pin_memory()
    b_w = torch.zeros(P, dtype=torch.float32).pin_memory()
    trace = phase_trace(0xE55100BB, 12 * T, E, k, 3 * T).reshape(12, P)
    for step in range(12):
        ids = dev(trace[step])
        w = dev(np.linspace(0.1, 1.0, P).astype(np.float32))
        slot_ids = torch.full((P,), -9, dtype=torch.int32, device="cuda")
        seq = 1000 + step
        m.cache_manage_gather(g.st, oracle.POLICIES[policy], ids, P, w, slot_ids, g.miss, g.n_miss, g.host_miss,
                              g.n_host, g.stats, store, slots, slab, sync, seq, bell, b_ids, b_slots, b_w)
        torch.cuda.synchronize()
        ro = o.manage(trace[step])
        np.testing.assert_array_equal(host(slot_ids), ro["slot_ids"])
        nm = int(host(g.n_miss)[0])
        np.testing.assert_array_equal(host(g.miss)[:2 * nm].reshape(-1, 2), ro["miss"])
        np.testing.assert_array_equal(host(g.stats), ro["stats"])
        b = bell.numpy()
        assert b[0] == seq and b[1] == nm and b[2] == len(ro["host_miss"]) and list(b[3:7]) == list(ro["stats"])
        np.testing.assert_array_equal(b_ids.numpy(), trace[step])
        np.testing.assert_array_equal(b_slots.numpy(), ro["slot_ids"])
        np.testing.assert_array_equal(b_w.numpy(), host(w))
        assert int(host(sync)[1]) == 0
        compare_state(g, o)
    s2e = host(g.s2e)[:S]
    for s_, e in enumerate(s2e):
        if e >= 0:
            np.testing.assert_array_equal(host(slots[s_]), store_h[e])


def compare_state(g, o):
    np.testing.assert_array_equal(host(g.e2s), o.e2s)
    if o.S:
        np.testing.assert_array_equal(host(g.s2e)[:o.S], o.s2e)
        np.testing.assert_array_equal(host(g.last)[:o.S].view(np.uint32), o.last)
        np.testing.assert_array_equal(host(g.freq)[:o.S].view(np.uint32), o.freq)
    assert int(host(g.step)[0]) == int(o.step[0])


@pytest.mark.parametrize("policy", ["lru", "lfu", "static"])
@pytest.mark.parametrize("E,S,T,k,dist", [(128, 32, 16, 8, "zipf"), (128, 32, 16, 8, "uniform"),
                                          (512, 192, 32, 10, "zipf"), (12, 1, 1, 1, "uniform"),
                                          (64, 64, 4, 8, "zipf"), (1000, 300, 40, 8, "zipf")])
def test_manage_matches_oracle_every_step(m, policy, E, S, T, k, dist):
    rng = np.random.default_rng(E * 31 + S)
    if dist == "zipf":
        seq = synth.zipf_ids(synth.key(E, 7, S), synth.key(E, 8, S), 30 * T, E, k, 0.8).reshape(30, T, k)
    else:
        seq = np.stack([np.stack([rng.choice(E, k, replace=False) for _ in range(T)]) for _ in range(30)])
    resident = list(rng.choice(E, S, replace=False)) if policy == "static" else None
    g = GpuCache(m, E, S, resident)
    o = oracle.Cache(E, S, policy, resident=resident)
    compare_state(g, o)
    for step in range(seq.shape[0]):
        rg = g.manage(policy, seq[step])
        ro = o.manage(seq[step])
        for key in ("slot_ids", "miss", "host_miss", "stats"):
            np.testing.assert_array_equal(rg[key], ro[key], err_msg=f"{key} at step {step}")
        compare_state(g, o)


def test_manage_empty_step_and_invalid_ids(m):
    g = GpuCache(m, 16, 4)
    o = oracle.Cache(16, 4, "lru")
    r = g.manage("lru", np.zeros(0, np.int32))
    ro = o.manage(np.zeros(0, np.int32))
    assert r["miss"].shape[0] == 0 and r["host_miss"].shape[0] == 0
    compare_state(g, o)


def test_pick_static_matches_oracle(m):
    li = synth.LayerInputs("c2", T=1024, with_store=False, step=10_000)
    zo = oracle.logits(li.x, 1, li.G)
    ids = oracle.topk(zo, 8)
    res = torch.empty(64, dtype=torch.int32, device="cuda")
    m.cache_pick_static(dev(ids.reshape(-1)), ids.size, 128, 64, res)
    np.testing.assert_array_equal(host(res), oracle.pick_static(ids, 128, 64))


def test_gather_copies_slabs_byte_exact(m):
    E, S, slab = 24, 6, 4096 + 256
    rng = np.random.default_rng(5)
    store = torch.empty((E, slab), dtype=torch.uint8, pin_memory=True)
    store.copy_(torch.from_numpy(rng.integers(0, 256, (E, slab), dtype=np.uint8)))
    slots = torch.zeros((S, slab), dtype=torch.uint8, device="cuda")
    g = GpuCache(m, E, S)
    o = oracle.Cache(E, S, "lru")
    o_slots = np.zeros((S, slab), np.uint8)
    for step in range(12):
        ids = rng.choice(E, 4, replace=False)
        rg = g.manage("lru", ids)
        ro = o.manage(ids)
        np.testing.assert_array_equal(rg["miss"], ro["miss"])
        m.cache_gather(g.miss, g.n_miss, S, store, slots, slab)
        oracle.gather(ro["miss"], store.numpy(), o_slots)
        np.testing.assert_array_equal(host(slots), o_slots)
    for s in range(S):
        e = int(o.s2e[s])
        if e >= 0:
            assert bytes(host(slots)[s]) == bytes(store.numpy()[e])


def test_gather_refuses_unpinned_host_memory(m):
    slab = 256
    store = torch.zeros((4, slab), dtype=torch.uint8)  # pageable
    slots = torch.zeros((2, slab), dtype=torch.uint8, device="cuda")
    miss = torch.zeros(4, dtype=torch.int32, device="cuda")
    n = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(m.MoeError) as e:
        m.cache_gather(miss, n, 2, store, slots, slab)
    assert e.value.code == m.MOE_E_ARG and "pinned" in str(e.value)
    # the refusal leaves no pending HIP error behind for the next caller
    assert float(torch.ones(4, device="cuda").sum()) == 4.0


# ------------------------------------------------------------------ FFN


def run_ffn(m, li, slot_ids, w, slot_store, S):
    T, k, H, I = li.T, li.k, li.H, li.I
    x = dev(li.x.view(np.int16) if li.x_dtype else li.x)
    ws_bytes = m.moe_ffn_workspace_bytes(T, k, S, li.w_type, H, I)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    y = torch.full((T, H), np.nan, dtype=torch.float32, device="cuda")
    m.moe_ffn_slots(x, li.x_dtype, dev(slot_ids.astype(np.int32)), dev(w), T, k, slot_store, li.slab, S, li.w_type,
                    H, I, y, ws, ws_bytes)
    return host(y)


def ffn_case(m, cfg, T, S=None, E=None, step=0, layer=0):
    li = synth.LayerInputs(cfg, T=T, E=E, step=step, layer=layer)
    z = oracle.logits(li.x, li.x_dtype, li.G)
    ids = oracle.topk(z, li.k)
    w = oracle.route_weights(z, ids)
    S = S if S is not None else li.c["S"]
    resident = li.c.get("resident") or oracle.pick_static(ids, li.E, S)
    c = oracle.Cache(li.E, S, "static", resident=resident)
    sl = c.manage(ids)["slot_ids"].reshape(ids.shape)
    slots = dev(li.store[np.asarray(resident)])
    _, yg, yh = oracle.layer(li.w_type, li.store, li.E, li.H, li.I, li.x, li.x_dtype, ids, w, sl)
    y = run_ffn(m, li, sl, w, slots, S)
    return li, ids, w, sl, y, yg, yh, slots


@pytest.mark.parametrize("cfg,T", [("c1", 16), ("c2", 1), ("c2", 8), ("c2", 64), ("c3", 16), ("c4", 1), ("c4", 32)])
def test_ffn_slots_matches_oracle(m, cfg, T):
    li, ids, w, sl, y, yg, yh, _ = ffn_case(m, cfg, T)
    assert_close(y, yg, li.w_type, f"{cfg} T={T}")
    none = np.all(sl < 0, axis=1)
    assert np.all(y[none] == 0) and not np.any(np.signbit(y[none]))


@pytest.mark.parametrize("w_type,H,I", [(1, 112, 144), (1, 1040, 784), (0, 80, 48), (2, 1040, 784),
                                        (2, 2320, 2080), (3, 1056, 544), (3, 224, 256), (3, 160, 1280),
                                        (2, 144, 48)])
def test_ffn_ragged_shapes(m, w_type, H, I):
    """Row tiles with a ragged tail and rows whose granules do not fill the waves;
    W8A8 with h rows longer than 2048 (quantised without holding the row in
    registers); 4-bit down rows of 17, 8 and 40 blocks (32-, 16- and 64-lane
    rows, eight per wave); int8 rows of 9 and 3 granules."""
    E, k, T, S = 12, 3, 11, 7
    rng = np.random.default_rng(H + I)
    x_dtype = 0 if w_type == 0 else 1
    x = synth.normal(synth.key(H, 1, I), (T, H), 1.0, x_dtype)
    store = synth.slabs(w_type, 1234 + w_type, 0, 0, E, H, I, 0.05)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.dirichlet(np.ones(k), T).astype(np.float32)
    resident = rng.choice(E, S, replace=False)
    e2s = np.full(E, -1, np.int32)
    e2s[resident] = np.arange(S)
    sl = e2s[ids]
    li = type("L", (), dict(T=T, k=k, H=H, I=I, E=E, x=x, x_dtype=x_dtype, w_type=w_type,
                            slab=store.shape[1]))
    _, yg, _ = oracle.layer(w_type, store, E, H, I, x, x_dtype, ids, w, sl)
    y = run_ffn(m, li, sl, w, dev(store[resident]), S)
    assert_close(y, yg, w_type, f"w{w_type} H={H} I={I}")


@pytest.mark.parametrize("w_type,T,H", [(1, 401, 112), (2, 401, 112), (2, 1500, 112), (0, 1700, 112),
                                        (2, 1400, 2112)])
def test_ffn_large_batch_sorted_picks(m, w_type, T, H):
    """Large batches on the row-streaming path: one sorting workgroup up to
    4096 picks, one per 1024 picks above (then x is quantised by a launch of
    its own, for H = 2112 without holding the row in registers)."""
    E, k, S, I = 12, 3, 7, 144
    rng = np.random.default_rng(17 + w_type)
    x_dtype = 0 if w_type == 0 else 1
    x = synth.normal(synth.key(99, 1, w_type), (T, H), 1.0, x_dtype)
    store = synth.slabs(w_type, 4321, 0, 0, E, H, I, 0.05)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.dirichlet(np.ones(k), T).astype(np.float32)
    resident = rng.choice(E, S, replace=False)
    e2s = np.full(E, -1, np.int32)
    e2s[resident] = np.arange(S)
    sl = e2s[ids]
    li = type("L", (), dict(T=T, k=k, H=H, I=I, E=E, x=x, x_dtype=x_dtype, w_type=w_type, slab=store.shape[1]))
    _, yg, _ = oracle.layer(w_type, store, E, H, I, x, x_dtype, ids, w, sl)
    y = run_ffn(m, li, sl, w, dev(store[resident]), S)
    assert_close(y, yg, w_type, f"w{w_type} T={T} k={k}")


@pytest.mark.parametrize("T,S,H,I", [(32, 5, 256, 128), (64, 32, 2048, 768), (200, 9, 384, 256), (600, 12, 256, 384),
                                     (40, 1, 128, 256)])
def test_ffn_int8_matrix_core_tiles(m, T, S, H, I):
    """W8A8 batches of 256 picks and more, on the int8 matrix-core tiles (32
    token rows per tile): one k-step and several, ragged tiles, several tiles
    per slot, non-resident picks, one slot, the 128-expert layer's shape at 64
    tokens, 1600 picks (one sorting workgroup with x's codes made in the same
    launch) and 4800 picks (the sort in two launches, x's codes in a launch of
    their own); repeat calls give the same bits."""
    E, k = max(16, 2 * S), 8
    rng = np.random.default_rng(T * 13 + S)
    x = synth.normal(synth.key(T, 8, S), (T, H), 1.0, 1)
    store = synth.slabs(2, 555 + H, 0, 0, E, H, I, 0.05)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.dirichlet(np.ones(k), T).astype(np.float32)
    resident = rng.choice(E, S, replace=False)
    e2s = np.full(E, -1, np.int32)
    e2s[resident] = np.arange(S)
    sl = e2s[ids]
    li = type("L", (), dict(T=T, k=k, H=H, I=I, E=E, x=x, x_dtype=1, w_type=2, slab=store.shape[1]))
    _, yg, _ = oracle.layer(2, store, E, H, I, x, 1, ids, w, sl)
    y = run_ffn(m, li, sl, w, dev(store[resident]), S)
    assert_close(y, yg, 2, f"int8 tiles T={T} S={S} H={H} I={I}")
    none = np.all(sl < 0, axis=1)
    assert np.all(y[none] == 0) and not np.any(np.signbit(y[none]))
    np.testing.assert_array_equal(run_ffn(m, li, sl, w, dev(store[resident]), S), y)


@pytest.mark.parametrize("T,k,S,H,I,mix", [(16, 8, 32, 2048, 768, "zipf"), (31, 8, 6, 256, 128, "hot"),
                                            (255, 1, 3, 128, 256, "hot"), (1, 8, 64, 2048, 768, "rand"),
                                            (5, 4, 16, 3072, 2048, "rand"), (7, 3, 8, 16, 16, "rand"),
                                            (9, 8, 700, 64, 1040, "rand")])
def test_ffn_int8_small_batches(m, T, k, S, H, I, mix):
    """W8A8 batches of fewer than 256 picks (the row-streaming kernels): the
    128-expert layer's 16-token Zipf batch; one slot picked by all 31 tokens
    (eight passes of four tokens over its rows); 255 one-pick tokens over 3
    slots; more slots than picks; rows of 3072 inputs and 2048 intermediate
    values; 16 x 16 experts; 700 slots with 1040-wide down rows.  Against the
    oracle, and every token's output is bit-identical to a batch of that token
    alone (int8 dots are exact, so a pick's result cannot depend on the
    batch)."""
    E = max(2 * S, 16, k + 4)
    rng = np.random.default_rng(T * 31 + S + H)
    x = synth.normal(synth.key(T, 9, S), (T, H), 1.0, 1)
    store = synth.slabs(2, 444 + H + I, 0, 0, E, H, I, 0.05)
    if mix == "zipf":
        ids = synth.zipf_ids(synth.key(T, 10), synth.key(T, 11), T, E, k, 0.8).astype(np.int32)
        resident = np.argsort(-np.bincount(ids.reshape(-1), minlength=E), kind="stable")[:S]
    elif mix == "hot":
        # expert 0 in every token's picks (k == 1: picks drawn from the first four experts)
        ids = (rng.integers(0, 4, size=(T, 1)) if k == 1 else
               np.stack([np.concatenate([[0], rng.choice(np.arange(1, E), k - 1, replace=False)]) for _ in range(T)]))
        ids = ids.astype(np.int32)
        resident = np.arange(S)
    else:
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        resident = rng.choice(E, S, replace=False)
    w = rng.dirichlet(np.ones(k), T).astype(np.float32)
    e2s = np.full(E, -1, np.int32)
    e2s[resident] = np.arange(S)
    sl = e2s[ids]
    assert T * k < 256 and (mix == "hot" or np.any(sl < 0))
    slots = dev(store[resident])
    li = type("L", (), dict(T=T, k=k, H=H, I=I, E=E, x=x, x_dtype=1, w_type=2, slab=store.shape[1]))
    _, yg, _ = oracle.layer(2, store, E, H, I, x, 1, ids, w, sl)
    y = run_ffn(m, li, sl, w, slots, S)
    assert_close(y, yg, 2, f"int8 small T={T} k={k} S={S} H={H} I={I}")
    none = np.all(sl < 0, axis=1)
    assert np.all(y[none] == 0) and not np.any(np.signbit(y[none]))
    np.testing.assert_array_equal(run_ffn(m, li, sl, w, slots, S), y)
    for t in sorted({0, T // 2, T - 1}):
        one = type("L", (), dict(T=1, k=k, H=H, I=I, E=E, x=x[t:t + 1], x_dtype=1, w_type=2, slab=store.shape[1]))
        np.testing.assert_array_equal(run_ffn(m, one, sl[t:t + 1], w[t:t + 1], slots, S), y[t:t + 1],
                                      err_msg=f"token {t} alone")


@pytest.mark.parametrize("w_type,T,k,S,H,I,mix", [(1, 8, 8, 64, 2048, 768, "zipf"), (1, 8, 8, 6, 2048, 768, "uniform"),
                                                   (1, 2, 8, 64, 2048, 768, "uniform"), (1, 64, 1, 5, 256, 128, "uniform"),
                                                   (1, 5, 8, 40, 112, 144, "uniform"), (0, 8, 8, 16, 64, 128, "uniform"),
                                                   (1, 6, 8, 200, 256, 128, "uniform"), (1, 4, 8, 16, 2048, 768, "cold")])
def test_ffn_small_batches(m, w_type, T, k, S, H, I, mix):
    """fp32 and bf16 batches of 2..64 picks, sorted by the one-wave sort: the
    128-expert layer's 8-token Zipf batch; 8 tokens over 6 slots (two passes
    of four over some slots); 64 one-pick tokens over 5 slots; ragged 112 x
    144 rows; fp32; 200 slots (the slot offsets summed 64 at a time); a batch
    with no resident pick.  Against the oracle, and bit-identical to the same
    tokens in a batch of more than 64 picks (sorted by k_group), padded with
    tokens whose picks all miss."""
    E = max(2 * S, 16, k + 4)
    rng = np.random.default_rng(T * 37 + S + H + w_type)
    x = synth.normal(synth.key(T, 12, S), (T, H), 1.0, 0 if w_type == 0 else 1)
    store = synth.slabs(w_type, 333 + H + I, 0, 0, E, H, I, 0.05)
    if mix == "zipf":
        ids = synth.zipf_ids(synth.key(T, 13), synth.key(T, 14), T, E, k, 0.8).astype(np.int32)
        resident = np.argsort(-np.bincount(ids.reshape(-1), minlength=E), kind="stable")[:S]
    else:
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        resident = rng.choice(E, S, replace=False)
    w = rng.dirichlet(np.ones(k), T).astype(np.float32)
    e2s = np.full(E, -1, np.int32)
    if mix != "cold":
        e2s[resident] = np.arange(S)
    sl = e2s[ids]
    assert 1 < T and T * k <= 64
    slots = dev(store[resident])
    li = type("L", (), dict(T=T, k=k, H=H, I=I, E=E, x=x, x_dtype=0 if w_type == 0 else 1, w_type=w_type,
                            slab=store.shape[1]))
    _, yg, _ = oracle.layer(w_type, store, E, H, I, x, li.x_dtype, ids, w, sl)
    y = run_ffn(m, li, sl, w, slots, S)
    assert_close(y, yg, w_type, f"small T={T} k={k} S={S} H={H} I={I} {mix}")
    none = np.all(sl < 0, axis=1)
    assert np.all(y[none] == 0) and not np.any(np.signbit(y[none]))
    # the same tokens followed by tokens whose picks all miss, past 64 picks: the workgroup sort
    n_pad = (64 - T * k) // k + 1
    xp = np.concatenate([x, x[:1].repeat(n_pad, axis=0)])
    slp = np.concatenate([sl, np.full((n_pad, k), -1, np.int32)])
    wp = np.concatenate([w, w[:1].repeat(n_pad, axis=0)])
    big = type("L", (), dict(T=T + n_pad, k=k, H=H, I=I, E=E, x=xp, x_dtype=li.x_dtype, w_type=w_type,
                             slab=store.shape[1]))
    assert (T + n_pad) * k > 64
    yp = run_ffn(m, big, slp, wp, slots, S)
    np.testing.assert_array_equal(yp[:T], y, err_msg="the same tokens sorted by the workgroup sort")
    assert np.all(yp[T:] == 0)


@pytest.mark.parametrize("w_type,H,I", [(0, 64, 128), (1, 2048, 768), (1, 112, 144), (2, 2048, 768), (3, 2048, 512),
                                        (3, 1056, 544)])
def test_ffn_one_token(m, w_type, H, I):
    """One-token batches: fp32, bf16 and 4-bit skip the pick sort (each
    gate/up and down workgroup takes one pick; 4-bit block sums made by those
    kernels), int8 keeps it.  Top-8 with some picks resident, a token whose
    picks share a slot (the same expert twice: each pick is still computed on
    its own), and a token with no resident pick (+0.0)."""
    E, k, S = 24, 8, 10
    rng = np.random.default_rng(H * 3 + I + w_type)
    x_dtype = 0 if w_type == 0 else 1
    store = synth.slabs(w_type, 4321 + w_type, 0, 0, E, H, I, 0.05)
    resident = rng.choice(E, S, replace=False)
    e2s = np.full(E, -1, np.int32)
    e2s[resident] = np.arange(S)
    slots = dev(store[resident])
    cold = np.setdiff1d(np.arange(E), resident)
    cases = [np.concatenate([resident[:5], cold[:3]]), np.array([resident[0]] * 2 + list(resident[1:3]) + list(cold[:4])),
             cold[:8]]
    for n, ids_row in enumerate(cases):
        ids = ids_row.astype(np.int32)[None, :]
        x = synth.normal(synth.key(H, 2, n), (1, H), 1.0, x_dtype)
        w = rng.dirichlet(np.ones(k), 1).astype(np.float32)
        sl = e2s[ids]
        li = type("L", (), dict(T=1, k=k, H=H, I=I, E=E, x=x, x_dtype=x_dtype, w_type=w_type, slab=store.shape[1]))
        _, yg, _ = oracle.layer(w_type, store, E, H, I, x, x_dtype, ids, w, sl)
        y = run_ffn(m, li, sl, w, slots, S)
        assert_close(y, yg, w_type, f"w{w_type} one token, case {n}")
        if n == 2:
            assert np.all(y == 0) and not np.any(np.signbit(y))
        np.testing.assert_array_equal(run_ffn(m, li, sl, w, slots, S), y)


@pytest.mark.parametrize("T,S", [(64, 24), (128, 40), (129, 40), (70, 1), (32, 24), (40, 12), (31, 24)])
def test_ffn_decode_sort_in_gemm(m, T, S):
    """bf16 decode batches of 256..1024 picks are grouped by slot inside the
    gate/up GEMM (no sort launch); 1032 picks go through the sort kernel, 248
    picks (31 tokens) through the row-streaming kernels.  Slots with several
    32-row tiles, non-resident picks, a single slot."""
    E, k, H, I = 40, 8, 256, 128
    rng = np.random.default_rng(T * 7 + S)
    x = synth.normal(synth.key(T, 1, S), (T, H), 1.0, 1)
    store = synth.slabs(1, 777, 0, 0, E, H, I, 0.05)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.dirichlet(np.ones(k), T).astype(np.float32)
    resident = rng.choice(E, S, replace=False)
    e2s = np.full(E, -1, np.int32)
    e2s[resident] = np.arange(S)
    sl = e2s[ids]
    li = type("L", (), dict(T=T, k=k, H=H, I=I, E=E, x=x, x_dtype=1, w_type=1, slab=store.shape[1]))
    _, yg, _ = oracle.layer(1, store, E, H, I, x, 1, ids, w, sl)
    y = run_ffn(m, li, sl, w, dev(store[resident]), S)
    assert_close(y, yg, 1, f"T={T} S={S}")
    none = np.all(sl < 0, axis=1)
    assert np.all(y[none] == 0) and not np.any(np.signbit(y[none]))
    np.testing.assert_array_equal(run_ffn(m, li, sl, w, dev(store[resident]), S), y)


def test_ffn_workspace_reused_across_calls(m):
    """One workspace for consecutive calls of different sizes (its counters clear themselves)."""
    big = ffn_case(m, "c2", 64)
    small = ffn_case(m, "c2", 8, step=3)
    S = 64
    ws_bytes = m.moe_ffn_workspace_bytes(64, 8, S, 1, 2048, 768)
    ws = torch.full((ws_bytes,), 0xAB, dtype=torch.uint8, device="cuda")
    for li, ids, w, sl, _, yg, _, slots in (big, small, big):
        x = dev(li.x.view(np.int16))
        y = torch.full((li.T, li.H), np.nan, dtype=torch.float32, device="cuda")
        m.moe_ffn_slots(x, 1, dev(sl.astype(np.int32)), dev(w), li.T, li.k, slots, li.slab, S, 1, li.H, li.I, y,
                        ws, ws_bytes)
        assert_close(host(y), yg, 1, f"reused workspace T={li.T}")


@pytest.mark.parametrize("T,S,H", [(300, 20, 256), (257, 24, 256), (1000, 17, 256), (600, 20, 384), (520, 18, 512),
                                   (700, 20, 1024)])
def test_ffn_prefill_grouped_gemm(m, T, S, H):
    """bf16 batches of >= 512 picks run on the MFMA grouped GEMMs: slots with
    more picks than one tile, ragged tiles, non-resident experts; from 4096
    picks the 128-row tiles, with four 32-row weight blocks per wave in the
    gate/up GEMM and, in the down GEMM, eight when H is a multiple of 256 (two
    and four 256-column tiles at H = 512 and 1024) and four otherwise.  The
    last tiles of the slots at T = 520 and 700 hold 1-32, 33-64, 65-96 and
    97-128 picks, so each count of staged 32-row token blocks runs."""
    E, k, I = 24, 8, 384
    rng = np.random.default_rng(T + S)
    x = synth.normal(synth.key(7, 1, T), (T, H), 1.0, 1)
    store = synth.slabs(1, 555, 0, 0, E, H, I, 0.05)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.dirichlet(np.ones(k), T).astype(np.float32)
    resident = rng.choice(E, S, replace=False)
    e2s = np.full(E, -1, np.int32)
    e2s[resident] = np.arange(S)
    sl = e2s[ids]
    li = type("L", (), dict(T=T, k=k, H=H, I=I, E=E, x=x, x_dtype=1, w_type=1, slab=store.shape[1]))
    _, yg, _ = oracle.layer(1, store, E, H, I, x, 1, ids, w, sl)
    y = run_ffn(m, li, sl, w, dev(store[resident]), S)
    assert_close(y, yg, 1, f"prefill T={T} S={S}")
    none = np.all(sl < 0, axis=1)
    assert np.all(y[none] == 0) and not np.any(np.signbit(y[none]))


@pytest.mark.parametrize("T", [511, 512])
def test_ffn_bf16_at_the_prefill_tile_switch(m, T):
    """4088 picks run on the decode-shaped tiles with fp32 partials, 4096 on
    the prefill-shaped tiles with bf16 partials; both against the oracle, on
    the same layer and the same first 511 tokens' picks."""
    E, k, H, I, S = 32, 8, 256, 384, 24
    rng = np.random.default_rng(4096)
    x = synth.normal(synth.key(13, 3, 512), (512, H), 1.0, 1)[:T]
    store = synth.slabs(1, 991, 0, 0, E, H, I, 0.05)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(512)]).astype(np.int32)[:T]
    w = rng.dirichlet(np.ones(k), 512).astype(np.float32)[:T]
    resident = rng.choice(E, S, replace=False)
    e2s = np.full(E, -1, np.int32)
    e2s[resident] = np.arange(S)
    sl = e2s[ids]
    li = type("L", (), dict(T=T, k=k, H=H, I=I, E=E, x=x, x_dtype=1, w_type=1, slab=store.shape[1]))
    _, yg, _ = oracle.layer(1, store, E, H, I, x, 1, ids, w, sl)
    y = run_ffn(m, li, sl, w, dev(store[resident]), S)
    assert_close(y, yg, 1, f"bf16 T={T}")
    none = np.all(sl < 0, axis=1)
    assert np.all(y[none] == 0) and not np.any(np.signbit(y[none]))


@pytest.mark.parametrize("T,k,E,S", [(4100, 1, 24, 20), (420, 10, 40, 30), (136, 32, 48, 36)])
def test_ffn_prefill_bf16_partials_other_k(m, T, k, E, S):
    """From 4096 picks the prefill-shaped GEMMs keep each pick's weighted
    row in bf16 and the reduction sums it in fp32 eight picks at a time: top-1
    (one pick per token), top-10 (a group of eight and a ragged group of two)
    and top-32 (four groups), with non-resident experts; every output against
    the oracle, tokens without a resident pick exactly +0."""
    H, I = 256, 384
    assert T * k >= 4096
    rng = np.random.default_rng(T * k)
    x = synth.normal(synth.key(11, 2, T), (T, H), 1.0, 1)
    store = synth.slabs(1, 777, 0, 0, E, H, I, 0.05)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.dirichlet(np.ones(k), T).astype(np.float32)
    resident = rng.choice(E, S, replace=False)
    e2s = np.full(E, -1, np.int32)
    e2s[resident] = np.arange(S)
    sl = e2s[ids]
    li = type("L", (), dict(T=T, k=k, H=H, I=I, E=E, x=x, x_dtype=1, w_type=1, slab=store.shape[1]))
    _, yg, _ = oracle.layer(1, store, E, H, I, x, 1, ids, w, sl)
    y = run_ffn(m, li, sl, w, dev(store[resident]), S)
    assert_close(y, yg, 1, f"prefill T={T} k={k}")
    none = np.all(sl < 0, axis=1)
    if k == 1:
        assert none.any()
    assert np.all(y[none] == 0) and not np.any(np.signbit(y[none]))


@pytest.mark.parametrize("T,S,skew", [(1200, 6, False), (1100, 8, True)])
def test_ffn_large_groups_256_row_tiles(m, T, S, skew):
    """Hundreds of picks per slot run on 256 x 256 tiles of eight waves:
    slots spanning several tiles with a ragged last one, a slot with few
    picks (waves without token rows), non-resident experts."""
    E, k, H, I = 8, 4, 256, 256
    rng = np.random.default_rng(T + S)
    x = synth.normal(synth.key(9, 1, T), (T, H), 1.0, 1)
    store = synth.slabs(1, 556, 0, 0, E, H, I, 0.05)
    p = np.array([0.3, 0.2, 0.2, 0.1, 0.1, 0.05, 0.04, 0.01]) if skew else np.ones(E) / E
    ids = np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    w = rng.dirichlet(np.ones(k), T).astype(np.float32)
    resident = rng.choice(E, S, replace=False)
    e2s = np.full(E, -1, np.int32)
    e2s[resident] = np.arange(S)
    sl = e2s[ids]
    assert T * k >= 4096 and T * k // S >= 384
    li = type("L", (), dict(T=T, k=k, H=H, I=I, E=E, x=x, x_dtype=1, w_type=1, slab=store.shape[1]))
    _, yg, _ = oracle.layer(1, store, E, H, I, x, 1, ids, w, sl)
    y = run_ffn(m, li, sl, w, dev(store[resident]), S)
    assert_close(y, yg, 1, f"large groups T={T} S={S}")
    none = np.all(sl < 0, axis=1)
    assert np.all(y[none] == 0) and not np.any(np.signbit(y[none]))



def test_ffn_large_groups_258_tiles(m):
    """Many 256 x 256 tiles on the large-group GEMMs: 129 resident slots of
    384 picks each (two tiles per slot, the second half full: 258 tiles, 33
    in each XCD's run of the tile list, 66 workgroups per XCD and GEMM), a
    non-resident expert, hidden 512 and intermediate 256.  Every token tile
    is checked through the tokens of its first and last pick (their outputs
    take every column tile of the tile), plus random tokens, against the
    oracle."""
    E, S, k, H, I = 130, 129, 2, 512, 256
    T = E * 384 // k
    t = np.arange(T)
    ids = np.stack([t % E, (t + 1 + (t // E) % (E - 1)) % E], axis=1).astype(np.int32)
    rng = np.random.default_rng(129)
    ids = ids[rng.permutation(T)]
    assert np.all(np.bincount(ids.ravel(), minlength=E) == 384) and np.all(ids[:, 0] != ids[:, 1])
    w = rng.dirichlet(np.ones(k), T).astype(np.float32)
    x = synth.normal(synth.key(11, 1, T), (T, H), 1.0, 1)
    store = synth.slabs(1, 557, 0, 0, E, H, I, 0.05)
    resident = np.setdiff1d(np.arange(E), [77])
    e2s = np.full(E, -1, np.int32)
    e2s[resident] = np.arange(S)
    sl = e2s[ids]
    li = type("L", (), dict(T=T, k=k, H=H, I=I, E=E, x=x, x_dtype=1, w_type=1, slab=store.shape[1]))
    y = run_ffn(m, li, sl, w, dev(store[resident]), S)
    assert np.all(np.isfinite(y))
    none = np.all(sl < 0, axis=1)
    assert np.all(y[none] == 0) and not np.any(np.signbit(y[none]))
    # a slot's picks in pick order, 256 to a tile: the first and last pick of each tile
    flat = sl.ravel()
    sample = set(rng.choice(T, 8, replace=False).tolist())
    for s in range(S):
        picks = np.flatnonzero(flat == s)
        for a in range(0, len(picks), 256):
            tile = picks[a:a + 256]
            sample.update((int(tile[0]) // k, int(tile[-1]) // k))
    for tok in sorted(sample):
        ref = np.zeros(H)
        for j in range(k):
            if sl[tok, j] >= 0:
                ref += w[tok, j] * oracle.expert(1, store[ids[tok, j]], H, I, x[tok], 1)
        assert_close(y[tok:tok + 1], ref[None, :].astype(np.float32), 1, f"many items token {tok}")


@functools.lru_cache(maxsize=1)
def prefill_inputs():
    """The 288-expert prefill layer's inputs (10.9 GB of slabs), made once per session."""
    li = synth.LayerInputs("c5")
    z = oracle.logits(li.x, 1, li.G)
    ids = oracle.topk(z, li.k)
    return li, ids, oracle.route_weights(z, ids)


@pytest.mark.parametrize("S", [288, 144])
def test_ffn_prefill_full_size_sampled(m, S):
    """The 288-expert prefill layer at full size (2048 tokens, hidden 4096,
    intermediate 1536): all resident, and the 144-slot variant whose misses
    return zero; sampled tokens against the oracle, the rest by property."""
    li, ids, w = prefill_inputs()
    if S == li.E:
        resident = np.arange(li.E)
    else:
        warm = synth.LayerInputs("c5", T=1024, step=10_000, with_store=False)
        resident = oracle.pick_static(oracle.topk(oracle.logits(warm.x, 1, warm.G), li.k), li.E, S)
    e2s = np.full(li.E, -1, np.int32)
    e2s[resident] = np.arange(S)
    sl = e2s[ids]
    y = run_ffn(m, li, sl, w, dev(li.store[resident]), S)
    assert np.all(np.isfinite(y))
    rng = np.random.default_rng(S)
    sample = np.concatenate([[0, li.T - 1], rng.choice(np.arange(1, li.T - 1), 10, replace=False)])
    for t in sample:
        ref = np.zeros(li.H)
        for j in range(li.k):
            if sl[t, j] >= 0:
                ref += w[t, j] * oracle.expert(1, li.store[ids[t, j]], li.H, li.I, li.x[t], 1)
        assert_close(y[t:t + 1], ref[None, :].astype(np.float32), 1, f"prefill S={S} token {t}")
    none = np.all(sl < 0, axis=1)
    assert np.all(y[none] == 0)


@pytest.mark.parametrize("S", [288, 144])
def test_ffn_prefill_16384_tokens_sampled(m, S):
    """The 288-expert layer at 16,384 tokens (about 455 picks per slot): the
    256 x 256 tiles with the full contractions (64 and 24 k-steps, the k walk
    rotated per slot for the 8 KiB gate/up rows); seeded random picks (eight
    distinct experts per token, Dirichlet weights), sampled tokens against the
    oracle, the tokens without a resident pick exactly zero."""
    li, _, _ = prefill_inputs()
    T, k, E, H, I = 16384, li.k, li.E, li.H, li.I
    rng = np.random.default_rng(16384 + S)
    x = synth.normal(synth.key(16384, 1, S), (T, H), 1.0, 1)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    w = rng.dirichlet(np.ones(k), T).astype(np.float32)
    resident = np.arange(E) if S == E else rng.choice(E, S, replace=False)
    e2s = np.full(E, -1, np.int32)
    e2s[resident] = np.arange(S)
    sl = e2s[ids]
    big = type("L", (), dict(T=T, k=k, H=H, I=I, E=E, x=x, x_dtype=1, w_type=1, slab=li.slab))
    y = run_ffn(m, big, sl, w, dev(li.store[resident]), S)
    assert np.all(np.isfinite(y))
    none = np.all(sl < 0, axis=1)
    assert np.all(y[none] == 0) and not np.any(np.signbit(y[none]))
    sample = np.concatenate([[0, T - 1], rng.choice(np.arange(1, T - 1), 10, replace=False)])
    for t in sample:
        ref = np.zeros(H)
        for j in range(k):
            if sl[t, j] >= 0:
                ref += w[t, j] * oracle.expert(1, li.store[ids[t, j]], H, I, x[t], 1)
        assert_close(y[t:t + 1], ref[None, :].astype(np.float32), 1, f"16384 tokens S={S} token {t}")


def test_ffn_many_tokens_on_one_slot(m):
    """More tokens on a slot than one pass holds (token chunks of 8)."""
    li = synth.LayerInputs("c2", T=37)
    k = li.k
    rng = np.random.default_rng(3)
    ids = np.stack([np.concatenate([[5], rng.choice(np.setdiff1d(np.arange(128), [5]), k - 1, replace=False)])
                    for _ in range(li.T)]).astype(np.int32)
    w = rng.dirichlet(np.ones(k), li.T).astype(np.float32)
    S = 16
    resident = np.arange(0, 32, 2)
    resident[2] = 5
    e2s = np.full(128, -1, np.int32)
    e2s[resident] = np.arange(S)
    sl = e2s[ids]
    _, yg, _ = oracle.layer(1, li.store, 128, li.H, li.I, li.x, 1, ids, w, sl)
    y = run_ffn(m, li, sl, w, dev(li.store[resident]), S)
    assert_close(y, yg, 1, "37 tokens on one slot")


def test_zero_return_is_exact(m):
    li = synth.LayerInputs("c2", T=8)
    w = np.full((8, 8), 0.125, np.float32)
    sl = np.full((8, 8), -1, np.int32)
    y = run_ffn(m, li, sl, w, dev(li.store[:4]), 4)
    assert np.all(y == 0) and not np.any(np.signbit(y))


def test_all_resident_any_permutation_bitwise(m):
    li = synth.LayerInputs("c1")
    z = oracle.logits(li.x, 0, li.G)
    ids = oracle.topk(z, 2)
    w = oracle.route_weights(z, ids)
    ident = run_ffn(m, li, ids, w, dev(li.store), 8)
    perm = np.random.default_rng(1).permutation(8)
    inv = np.argsort(perm)  # slot s holds expert perm[s]
    y = run_ffn(m, li, inv[ids], w, dev(li.store[perm]), 8)
    np.testing.assert_array_equal(y, ident)
    yf, _, _ = oracle.layer(0, li.store, 8, 64, 128, li.x, 0, ids, w)
    assert_close(ident, yf, 0, "all resident vs no cache")


def test_ffn_deterministic(m):
    li, ids, w, sl, y, yg, yh, slots = ffn_case(m, "c2", 64)
    y2 = run_ffn(m, li, sl, w, slots, 64)
    np.testing.assert_array_equal(y, y2)


# ---------------------------------------------------------- whole layer


@pytest.mark.parametrize("cfg,T", [("c1", 16), ("c2", 8), ("c2", 64)])
def test_layer_step_two_passes_sum_to_oracle(m, cfg, T):
    from expert_vram_slot_amd.layer import SlotLayer
    li = synth.LayerInputs(cfg, T=T)
    c = li.c
    S = c["S"]
    zo = oracle.logits(li.x, li.x_dtype, li.G)
    ids_o = oracle.topk(zo, li.k)
    w_o = oracle.route_weights(zo, ids_o)
    yf, _, _ = oracle.layer(li.w_type, li.store, li.E, li.H, li.I, li.x, li.x_dtype, ids_o, w_o)
    if cfg == "c1":
        resident = np.array(c["resident"], np.int32)
    else:
        warm = synth.LayerInputs(cfg, T=1024, step=10_000, with_store=False)
        resident = oracle.pick_static(oracle.topk(oracle.logits(warm.x, 1, warm.G), li.k), li.E, S)
    host_store = torch.empty(li.store.shape, dtype=torch.uint8, pin_memory=True)
    host_store.copy_(torch.from_numpy(li.store))
    slots = dev(li.store[resident])
    G = dev(li.G.view(np.int16) if li.x_dtype else li.G)
    L = SlotLayer(E=li.E, k=li.k, H=li.H, I=li.I, S=S, w_type=li.w_type, T_max=T, policy="static",
                  host_store=host_store, slot_store=slots, G=G, n_threads=8)
    L.init_cache(dev(resident))
    x = dev(li.x.view(np.int16) if li.x_dtype else li.x)
    y = host(L.step(x, T))
    np.testing.assert_array_equal(host(L.ids)[:T * li.k].reshape(T, li.k), ids_o)
    assert_close(y, yf, li.w_type, f"{cfg} layer")
    st = host(L.stats)
    assert st[3] == len(set(ids_o.reshape(-1).tolist()) - set(resident.tolist()))


# ---------------------------------------------------------- layer stack


@functools.lru_cache(maxsize=1)
def stack_layers(n_layers=3):
    """Layers of the 48 x 512-expert 4-bit stack (full per-layer shape) with
    their brightness profiles, hot/resident sets and stores."""
    out = []
    for l in range(n_layers):
        li = synth.LayerInputs("c4", layer=l, T=1)
        b = synth.dirichlet(synth.key(li.base, synth.TAG_B, l), li.E, li.c["alpha"])
        resident = np.lexsort((np.arange(li.E), -b))[:li.c["S"]].astype(np.int32)
        out.append((li, b, resident))
    return out


@pytest.mark.parametrize("T", [1, 32])
def test_stack_teacher_forced_per_layer(m, T):
    """Three layers of the 4-bit stack with the graded bias and 192 resident
    experts per layer, run as a stack; every layer checked on the inputs the
    GPU gave it: ids and slots bitwise, weights fp32, output 4-bit tolerance,
    the residual stream bitwise."""
    from expert_vram_slot_amd.layer import SlotStack
    layers = stack_layers()
    li0 = layers[0][0]
    E, k, H, I, S, cap = li0.E, li0.k, li0.H, li0.I, li0.c["S"], li0.c["cap"]
    specs = []
    for li, b, resident in layers:
        bias = torch.empty(E, dtype=torch.float32, device="cuda")
        m.moe_bias_table(dev(b), E, S, cap, bias)
        specs.append(dict(host_store=torch.from_numpy(li.store).pin_memory(), slot_store=dev(li.store[resident]),
                          G=dev(li.G.view(np.int16)), bias=bias, resident=dev(resident)))
    stack = SlotStack(E=E, k=k, H=H, I=I, S=S, w_type=3, T_max=T, layers=specs)
    x0 = synth.LayerInputs("c4", layer=0, T=T, with_store=False).x
    trace = []
    out = host(stack.step(dev(x0.view(np.int16)), T, trace=trace)).view(np.uint16)
    assert np.array_equal(host(trace[0][0]).view(np.uint16), x0)
    for l, ((li, b, resident), (xl, ids, sl, w, y)) in enumerate(zip(layers, trace)):
        xl = host(xl).view(np.uint16)
        z = oracle.logits(xl, 1, li.G)
        ids_o = oracle.topk(z, k, oracle.bias_table(b, S, cap))
        w_o = oracle.route_weights(z, ids_o)
        np.testing.assert_array_equal(host(ids).reshape(T, k), ids_o, err_msg=f"layer {l} ids")
        e2s = np.full(E, -1, np.int32)
        e2s[resident] = np.arange(S)
        np.testing.assert_array_equal(host(sl).reshape(T, k), e2s[ids_o], err_msg=f"layer {l} slots")
        assert_close(host(w).reshape(T, k), w_o, 0, f"layer {l} weights")
        yf, _, _ = oracle.layer(3, li.store, E, H, I, xl, 1, ids_o, w_o, e2s[ids_o])
        y = host(y)
        assert_close(y, yf, 3, f"layer {l} output")
        nxt = oracle.residual(xl, 1, y)
        got = host(trace[l + 1][0]).view(np.uint16) if l + 1 < len(trace) else out
        np.testing.assert_array_equal(got, nxt, err_msg=f"layer {l} residual")


def test_residual_matches_oracle(m):
    x = synth.normal(synth.key(5, 1), (33, 2048), 1.0, 1)
    y = synth.normal(synth.key(5, 2), (33, 2048), 0.5, 0)
    xo = torch.empty((33, 2048), dtype=torch.int16, device="cuda")
    m.moe_residual(dev(x.view(np.int16)), 1, dev(y), xo, 33, 2048)
    np.testing.assert_array_equal(host(xo).view(np.uint16), oracle.residual(x, 1, y))
    xf = synth.normal(synth.key(5, 3), (7, 64), 1.0, 0)
    xfo = torch.empty((7, 64), dtype=torch.float32, device="cuda")
    m.moe_residual(dev(xf), 0, dev(y[:7, :64].copy()), xfo, 7, 64)
    np.testing.assert_array_equal(host(xfo), oracle.residual(xf, 0, y[:7, :64]))


# ------------------------------------------------------- native step driver


def _layer_spec(li, resident, policy="static", S=None):
    S = len(resident) if S is None else S
    slots = torch.zeros((max(S, 1), li.slab), dtype=torch.uint8, device="cuda")
    if policy == "static":
        slots[:len(resident)] = dev(li.store[np.asarray(resident)])
    return dict(host_store=torch.from_numpy(li.store).pin_memory(), slot_store=slots,
                G=dev(li.G.view(np.int16) if li.x_dtype else li.G), bias=None,
                resident=dev(np.asarray(resident, np.int32)) if policy == "static" else None, policy=policy)


@pytest.mark.parametrize("cfg,T", [("c1", 16), ("c2", 8), ("c2", 64)])
def test_native_layer_step_equals_python_orchestration(m, cfg, T):
    """moe_layer_step issues the same kernels as SlotLayer: identical bits, and the oracle's layer."""
    from expert_vram_slot_amd.layer import NativeStack, SlotLayer
    li = synth.LayerInputs(cfg, T=T)
    z = oracle.logits(li.x, li.x_dtype, li.G)
    ids = oracle.topk(z, li.k)
    w = oracle.route_weights(z, ids)
    S = li.c["S"]
    resident = li.c.get("resident") or oracle.pick_static(ids, li.E, S)
    spec = _layer_spec(li, resident)
    nat = NativeStack(E=li.E, k=li.k, H=li.H, I=li.I, S=S, w_type=li.w_type, T_max=T, layers=[spec])
    x = dev(li.x.view(np.int16) if li.x_dtype else li.x)
    y_nat = host(nat.layer_step(0, x, T))
    L = SlotLayer(E=li.E, k=li.k, H=li.H, I=li.I, S=S, w_type=li.w_type, T_max=T, policy="static",
                  host_store=spec["host_store"], slot_store=spec["slot_store"], G=spec["G"])
    L.init_cache(spec["resident"])
    y_py = host(L.step(x, T))
    np.testing.assert_array_equal(y_nat, y_py)
    yf, _, _ = oracle.layer(li.w_type, li.store, li.E, li.H, li.I, li.x, li.x_dtype, ids, w)
    assert_close(y_nat, yf, li.w_type, f"native {cfg} T={T}")
    hits, distinct, gathered, nhost = nat.stats()
    e2s = np.full(li.E, -1, np.int32)
    e2s[np.asarray(resident)] = np.arange(S)
    assert hits == int(np.sum(e2s[ids] >= 0)) and gathered == 0
    nat.close()


def test_native_dynamic_cache_steps(m):
    """A W8A8 layer with 32 LRU slots from empty, Zipf picks given: each step
    of the native driver equals the Python orchestration bit for bit, and the
    oracle's layer with the oracle's cache state machine."""
    from expert_vram_slot_amd.layer import NativeStack, SlotLayer
    li = synth.LayerInputs("c3", T=16)
    E, k, S, T = li.E, li.k, 32, 16
    steps = 6
    seq = synth.zipf_ids(synth.key(li.base, synth.TAG_ZIPF_PERM), synth.key(li.base, synth.TAG_ZIPF_DRAW),
                         steps * T, E, k, 0.8).reshape(steps, T, k)
    spec = _layer_spec(li, [], policy="lru", S=S)
    spec_py = dict(spec, slot_store=torch.zeros_like(spec["slot_store"]))
    nat = NativeStack(E=E, k=k, H=li.H, I=li.I, S=S, w_type=li.w_type, T_max=T, layers=[spec])
    L = SlotLayer(E=E, k=k, H=li.H, I=li.I, S=S, w_type=li.w_type, T_max=T, policy="lru",
                  host_store=spec_py["host_store"], slot_store=spec_py["slot_store"], G=spec_py["G"])
    L.init_cache(None)
    cache = oracle.Cache(E, S, "lru")
    for st in range(steps):
        x_np = synth.normal(synth.key(li.base, synth.TAG_X, 0, 100 + st), (T, li.H), 1.0, 1)
        x = dev(x_np.view(np.int16))
        ids_in = dev(seq[st])
        y_nat = host(nat.layer_step(0, x, T, ids_in=ids_in))
        y_py = host(L.step(x, T, ids_in=ids_in))
        np.testing.assert_array_equal(y_nat, y_py, err_msg=f"step {st}")
        z = oracle.logits(x_np, 1, li.G)
        w = oracle.route_weights(z, seq[st])
        sl = cache.manage(seq[st])["slot_ids"].reshape(T, k)
        yf, _, _ = oracle.layer(li.w_type, li.store, E, li.H, li.I, x_np, 1, seq[st], w, sl)
        assert_close(y_nat, yf, li.w_type, f"dynamic step {st}")
    np.testing.assert_array_equal(host(nat.e2s(0)), cache.e2s)
    nat.close()


def test_native_dynamic_cache_steps_without_host_pass(m):
    """The native driver without the host pass runs the cache step and the
    gather as two launches: bit for bit the Python orchestration's GPU pass,
    which is the oracle's y_gpu (resident picks only)."""
    from expert_vram_slot_amd.layer import NativeStack, SlotLayer
    li = synth.LayerInputs("c3", T=16)
    E, k, S, T = li.E, li.k, 32, 16
    steps = 4
    seq = synth.zipf_ids(synth.key(li.base, synth.TAG_ZIPF_PERM), synth.key(li.base, synth.TAG_ZIPF_DRAW, 1),
                         steps * T, E, k, 0.8).reshape(steps, T, k)
    spec = _layer_spec(li, [], policy="lru", S=S)
    spec_py = dict(spec, slot_store=torch.zeros_like(spec["slot_store"]))
    nat = NativeStack(E=E, k=k, H=li.H, I=li.I, S=S, w_type=li.w_type, T_max=T, layers=[spec])
    L = SlotLayer(E=E, k=k, H=li.H, I=li.I, S=S, w_type=li.w_type, T_max=T, policy="lru",
                  host_store=spec_py["host_store"], slot_store=spec_py["slot_store"], G=spec_py["G"])
    L.init_cache(None)
    cache = oracle.Cache(E, S, "lru")
    for st in range(steps):
        x_np = synth.normal(synth.key(li.base, synth.TAG_X, 0, 200 + st), (T, li.H), 1.0, 1)
        x = dev(x_np.view(np.int16))
        ids_in = dev(seq[st])
        y_nat = host(nat.layer_step(0, x, T, ids_in=ids_in, host_pass=False))
        y_py = host(L.step(x, T, ids_in=ids_in, host_pass=False))
        np.testing.assert_array_equal(y_nat, y_py, err_msg=f"step {st}")
        z = oracle.logits(x_np, 1, li.G)
        w = oracle.route_weights(z, seq[st])
        sl = cache.manage(seq[st])["slot_ids"].reshape(T, k)
        _, yg, _ = oracle.layer(li.w_type, li.store, E, li.H, li.I, x_np, 1, seq[st], w, sl)
        assert_close(y_nat, yg, li.w_type, f"gpu pass, step {st}")
    np.testing.assert_array_equal(host(spec["slot_store"]), host(spec_py["slot_store"]))
    nat.close()


def test_native_gather_give_up_is_reported(m):
    """A copying workgroup of the fused cache step that stops waiting for the
    managing one copies nothing; the step must then fail loudly rather than
    compute on stale slots.  Forced from the host with a wait of zero polls
    (every workgroup still runs to its end, nothing hangs): the step returns
    an error naming the incomplete gather.  With the default wait back and
    the cache set again, the same step matches the oracle."""
    from expert_vram_slot_amd.layer import NativeStack
    li = synth.LayerInputs("c3", T=16)
    E, k, S, T = li.E, li.k, 32, 16
    ids_np = synth.zipf_ids(synth.key(li.base, synth.TAG_ZIPF_PERM), synth.key(li.base, synth.TAG_ZIPF_DRAW, 2),
                            T, E, k, 0.8)
    spec = _layer_spec(li, [], policy="lru", S=S)
    nat = NativeStack(E=E, k=k, H=li.H, I=li.I, S=S, w_type=li.w_type, T_max=T, layers=[spec])
    x_np = synth.normal(synth.key(li.base, synth.TAG_X, 0, 300), (T, li.H), 1.0, 1)
    x, ids_in = dev(x_np.view(np.int16)), dev(ids_np)
    default = m.moe_fused_spin_limit(-1)
    assert default > 0
    prev = m.moe_fused_spin_limit(0)
    try:
        with pytest.raises(m.MoeError) as ei:
            nat.layer_step(0, x, T, ids_in=ids_in)
        assert ei.value.code == m.MOE_E_HIP and "gather of this step is incomplete" in str(ei.value)
    finally:
        m.moe_fused_spin_limit(prev)
    torch.cuda.synchronize()
    assert m.moe_fused_spin_limit(-1) == default
    nat.init_cache(0, None)
    spec["slot_store"].zero_()
    y = host(nat.layer_step(0, x, T, ids_in=ids_in))
    z = oracle.logits(x_np, 1, li.G)
    w = oracle.route_weights(z, ids_np)
    yf, _, _ = oracle.layer(li.w_type, li.store, E, li.H, li.I, x_np, 1, ids_np, w)
    assert_close(y, yf, li.w_type, "step after the reported give-up")
    nat.close()


@functools.lru_cache(maxsize=1)
def prefill_144_host():
    """The 144-slot variant of the 288-expert layer: its resident set (the 144
    most-picked experts of a 1024-token profile batch) and the pinned host
    store of all 288 experts."""
    li, _, _ = prefill_inputs()
    warm = synth.LayerInputs("c5", T=1024, step=10_000, with_store=False)
    resident = oracle.pick_static(oracle.topk(oracle.logits(warm.x, 1, warm.G), li.k), li.E, 144)
    return resident.astype(np.int32), torch.from_numpy(li.store).pin_memory()


@pytest.mark.parametrize("mode", ["cpu", "streamed"])
def test_native_prefill_144_slots_with_host_misses(m, mode):
    """The full 288-expert layer at 2048 tokens with 144 experts resident and
    the other 144 served by the step itself, either by the CPU lane (forced)
    or, as the switch picks at this batch size (about 57 picks per
    non-resident expert), streamed through the GPU's staging slots: the whole
    layer's output on sampled tokens against the oracle."""
    from expert_vram_slot_amd.layer import NativeStack
    li, ids, w = prefill_inputs()
    resident, host_store = prefill_144_host()
    S, T = 144, li.T
    spec = dict(host_store=host_store, slot_store=dev(li.store[resident]), G=dev(li.G.view(np.int16)), bias=None,
                resident=dev(resident))
    nat = NativeStack(E=li.E, k=li.k, H=li.H, I=li.I, S=S, w_type=1, T_max=T, layers=[spec])
    if mode == "cpu":
        nat.set_stream_threshold(-1)
    y = host(nat.layer_step(0, dev(li.x.view(np.int16)), T))
    assert nat.last_host_mode() == (1 if mode == "cpu" else 2)
    hits, distinct, gathered, nhost = nat.stats()
    e2s = np.full(li.E, -1, np.int32)
    e2s[resident] = np.arange(S)
    assert hits == int(np.sum(e2s[ids] >= 0)) and gathered == 0 and nhost == len(set(ids[e2s[ids] < 0].tolist()))
    assert np.all(np.isfinite(y))
    rng = np.random.default_rng(144)
    sample = np.concatenate([[0, T - 1], rng.choice(np.arange(1, T - 1), 6, replace=False)])
    for t in sample:
        ref = np.zeros(li.H)
        for j in range(li.k):
            ref += w[t, j] * oracle.expert(1, li.store[ids[t, j]], li.H, li.I, li.x[t], 1)
        assert_close(y[t:t + 1], ref[None, :].astype(np.float32), 1, f"{mode} token {t}")
    nat.close()
    del spec
    torch.cuda.empty_cache()


def test_native_switch_at_its_threshold(m):
    """The big-batch switch compares the step's host picks with the
    threshold times its host experts: with the threshold at the step's own
    ratio (rounded down) the misses stream, one above it the CPU lane runs.
    The 128-expert bf16 layer at 256 tokens (a step with a staging ring), 64
    experts resident; both lanes' outputs against the oracle on sampled
    tokens, and a step the default threshold sends to the CPU lane."""
    from expert_vram_slot_amd.layer import NativeStack
    T = 256
    li = synth.LayerInputs("c2", T=T)
    E, k, H, I, S = li.E, li.k, li.H, li.I, 64
    z = oracle.logits(li.x, 1, li.G)
    ids = oracle.topk(z, k)
    w = oracle.route_weights(z, ids)
    resident = np.arange(0, E, 2).astype(np.int32)
    e2s = np.full(E, -1, np.int32)
    e2s[resident] = np.arange(S)
    host_ids = ids[e2s[ids] < 0]
    ratio = len(host_ids) / len(set(host_ids.tolist()))
    assert 8 < ratio < 40  # the default threshold keeps this step on the CPU lane
    spec = dict(host_store=torch.from_numpy(li.store).pin_memory(), slot_store=dev(li.store[resident]),
                G=dev(li.G.view(np.int16)), bias=None, resident=dev(resident))
    nat = NativeStack(E=E, k=k, H=H, I=I, S=S, w_type=1, T_max=T, layers=[spec])
    x = dev(li.x.view(np.int16))
    rng = np.random.default_rng(256)
    sample = np.concatenate([[0, T - 1], rng.choice(np.arange(1, T - 1), 6, replace=False)])
    for thr, mode in ((None, 1), (int(np.floor(ratio)), 2), (int(np.floor(ratio)) + 1, 1)):
        if thr is not None:
            nat.set_stream_threshold(thr)
        y = host(nat.layer_step(0, x, T))
        assert nat.last_host_mode() == mode, f"threshold {thr}, {ratio:.2f} host picks per host expert"
        assert np.all(np.isfinite(y))
        for t in sample:
            ref = np.zeros(H)
            for j in range(k):
                ref += w[t, j] * oracle.expert(1, li.store[ids[t, j]], H, I, li.x[t], 1)
            assert_close(y[t:t + 1], ref[None, :].astype(np.float32), 1, f"threshold {thr} token {t}")
    nat.close()


@pytest.mark.parametrize("T", [1, 32])
def test_native_stack_equals_python_stack(m, T):
    from expert_vram_slot_amd.layer import NativeStack, SlotStack
    layers = stack_layers()
    li0 = layers[0][0]
    E, k, H, I, S, cap = li0.E, li0.k, li0.H, li0.I, li0.c["S"], li0.c["cap"]
    specs = []
    for li, b, resident in layers:
        bias = torch.empty(E, dtype=torch.float32, device="cuda")
        m.moe_bias_table(dev(b), E, S, cap, bias)
        specs.append(dict(host_store=torch.from_numpy(li.store).pin_memory(), slot_store=dev(li.store[resident]),
                          G=dev(li.G.view(np.int16)), bias=bias, resident=dev(resident)))
    x0 = dev(synth.LayerInputs("c4", layer=0, T=T, with_store=False).x.view(np.int16))
    py = SlotStack(E=E, k=k, H=H, I=I, S=S, w_type=3, T_max=T, layers=specs)
    out_py = host(py.step(x0, T))
    nat = NativeStack(E=E, k=k, H=H, I=I, S=S, w_type=3, T_max=T, layers=specs)
    out_nat = host(nat.step(x0, T))
    np.testing.assert_array_equal(out_nat, out_py)
    out_nat2 = host(nat.step(x0, T))
    np.testing.assert_array_equal(out_nat2, out_py)
    nat.close()


# ------------------------------------------------------------- edge cases


def _small_layer(name, T, E, H, k, x_dtype, seed):
    """Router inputs of a synthetic layer (x ~ N(0, 1), G ~ N(0, 0.05))."""
    x = synth.normal(synth.key(seed, 1, T), (T, H), 1.0, x_dtype)
    G = synth.normal(synth.key(seed, 2, E), (E, H), 0.05, x_dtype)
    return type(name, (), dict(T=T, H=H, E=E, k=k, x=x, G=G, x_dtype=x_dtype))


@pytest.mark.parametrize("E,k", [(4096, 32), (4096, 1), (33, 32), (32, 32)])
def test_route_limits_of_experts_and_top_k(m, E, k):
    """The ABI's limits: 4,096 experts, top-32; top-1; k = E (every expert
    picked, in rank order).  Ids bitwise against the oracle on the GPU's own
    logits and at this seed, weights within fp32 tolerance, both router forms."""
    li = _small_layer("L", 6, E, 64, k, 0, 4000 + E + k)
    check_route(m, li)
    ids_f, w_f, _ = gpu_route(m, li, with_logits=False)
    z = oracle.logits(li.x, 0, li.G)
    np.testing.assert_array_equal(ids_f, oracle.topk(z, k))
    np.testing.assert_allclose(w_f, oracle.route_weights(z, ids_f), rtol=2e-6, atol=1e-9)
    if k == E:
        np.testing.assert_allclose(w_f.sum(axis=1), 1.0, rtol=1e-5)


@pytest.mark.parametrize("policy", ["lru", "lfu"])
def test_manage_limits_of_experts_and_slots(m, policy):
    """4,096 experts over 1,024 slots (the ABI's limits), steps of 2,048 ids
    drawn Zipf(0.8), overflow into the host list on every step: each step's
    slot ids, miss list, host list, counters and state bitwise against the
    oracle."""
    E, S, k = 4096, 1024, 32
    g = GpuCache(m, E, S)
    o = oracle.Cache(E, S, policy)
    for st in range(4):
        ids = synth.zipf_ids(synth.key(0xE5510F00, 7, st), synth.key(0xE5510F00, 8, st), 64, E, k, 0.8)
        rg, ro = g.manage(policy, ids), o.manage(ids)
        for key in ("slot_ids", "miss", "host_miss", "stats"):
            np.testing.assert_array_equal(rg[key], ro[key], err_msg=f"{policy} step {st} {key}")
    np.testing.assert_array_equal(host(g.e2s), o.e2s)
    np.testing.assert_array_equal(host(g.s2e), o.s2e)


@pytest.mark.parametrize("w_type,k", [(0, 1), (1, 1), (2, 1), (3, 1), (0, 32), (1, 32), (2, 32), (3, 32)])
def test_ffn_top1_and_top32(m, w_type, k):
    """One pick per token and 32 picks per token (the ABI's limit; 288 picks
    take the int8 tiles for W8A8), every weight format, a third of the
    experts resident."""
    E, S, T, H, I = 48, 16, 9, 256, 128
    rng = np.random.default_rng(w_type * 100 + k)
    x_dtype = 0 if w_type == 0 else 1
    x = synth.normal(synth.key(k, 3, w_type), (T, H), 1.0, x_dtype)
    store = synth.slabs(w_type, 8800 + w_type, 0, 0, E, H, I, 0.05)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.dirichlet(np.ones(k), T).astype(np.float32)
    resident = rng.choice(E, S, replace=False)
    e2s = np.full(E, -1, np.int32)
    e2s[resident] = np.arange(S)
    sl = e2s[ids]
    li = type("L", (), dict(T=T, k=k, H=H, I=I, E=E, x=x, x_dtype=x_dtype, w_type=w_type, slab=store.shape[1]))
    _, yg, _ = oracle.layer(w_type, store, E, H, I, x, x_dtype, ids, w, sl)
    y = run_ffn(m, li, sl, w, dev(store[resident]), S)
    assert_close(y, yg, w_type, f"w{w_type} k={k}")


@pytest.mark.parametrize("T", [4, 40, 600])
def test_ffn_1024_slots(m, T):
    """The ABI's largest slot count (1,024 slots of 1,200 experts, bf16, H = I
    = 128) at 32 picks (the one-wave sort, its offsets over 16 groups of 64
    slots), 320 picks (matrix-core tiles sorted inside the gate/up kernel) and
    4,800 picks (prefill tiles, the multi-workgroup sort), a sixth of the
    experts not resident.  Against the oracle."""
    E, S, k, H, I = 1200, 1024, 8, 128, 128
    rng = np.random.default_rng(1024 + T)
    x = synth.normal(synth.key(T, 21, S), (T, H), 1.0, 1)
    store = synth.slabs(1, 1024, 0, 0, E, H, I, 0.05)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.dirichlet(np.ones(k), T).astype(np.float32)
    resident = rng.choice(E, S, replace=False)
    e2s = np.full(E, -1, np.int32)
    e2s[resident] = np.arange(S)
    sl = e2s[ids]
    li = type("L", (), dict(T=T, k=k, H=H, I=I, E=E, x=x, x_dtype=1, w_type=1, slab=store.shape[1]))
    _, yg, _ = oracle.layer(1, store, E, H, I, x, 1, ids, w, sl)
    y = run_ffn(m, li, sl, w, dev(store[resident]), S)
    assert_close(y, yg, 1, f"1024 slots T={T}")
    none = np.all(sl < 0, axis=1)
    assert np.all(y[none] == 0) and not np.any(np.signbit(y[none]))


def test_empty_batch_is_a_no_op(m):
    """T = 0 tokens through every entry point that takes a batch: each returns
    success and leaves its outputs as they were; the native step too."""
    from expert_vram_slot_amd.layer import NativeStack
    li = synth.LayerInputs("c1")
    E, k, H, I, S = li.E, li.k, li.H, li.I, 4
    x = dev(li.x)
    G = dev(li.G)
    sentinel = -12345
    ids = torch.full((4, k), sentinel, dtype=torch.int32, device="cuda")
    w = torch.full((4, k), 7.0, dtype=torch.float32, device="cuda")
    m.moe_route(x, 0, G, None, None, 0, H, E, k, ids, w, None)
    g = GpuCache(m, E, S, [0, 1, 2, 3])
    slot_ids = torch.full((4 * k,), sentinel, dtype=torch.int32, device="cuda")
    m.cache_manage(g.st, oracle.POLICIES["lru"], ids, 0, slot_ids, g.miss, g.n_miss, g.host_miss, g.n_host, g.stats)
    slots = dev(li.store[:S])
    y = torch.full((4, H), 7.0, dtype=torch.float32, device="cuda")
    wsb = m.moe_ffn_workspace_bytes(1, k, S, 0, H, I)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    m.moe_ffn_slots(x, 0, slot_ids, w, 0, k, slots, li.slab, S, 0, H, I, y, ws, wsb)
    m.moe_ffn_slots_noalloc(x, 0, slot_ids, w, 0, k, slots, li.slab, S, 0, H, I, y)
    m.moe_combine(y, y, 0, H)
    xo = torch.full((4, H), 7.0, dtype=torch.float32, device="cuda")
    m.moe_residual(x, 0, y, xo, 0, H)
    spec = _layer_spec(li, [0, 1, 2, 3])
    nat = NativeStack(E=E, k=k, H=H, I=I, S=S, w_type=0, T_max=4, layers=[spec])
    nat.y.fill_(7.0)
    nat.layer_step(0, x, 0)
    torch.cuda.synchronize()
    assert torch.all(ids == sentinel) and torch.all(w == 7.0) and torch.all(slot_ids == sentinel)
    assert torch.all(y == 7.0) and torch.all(xo == 7.0) and torch.all(nat.y == 7.0)
    assert int(host(g.step)[0]) == 1  # an empty cache step still counts as a step (oracle: same)
    o = oracle.Cache(E, S, "lru", [0, 1, 2, 3])
    o.manage(np.zeros(0, np.int32))
    assert int(o.step[0]) == 1
    nat.close()
