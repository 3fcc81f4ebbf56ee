"""moe_ffn_slots_noalloc (workspace in a static device array) against
moe_ffn_slots (workspace passed in): identical bits, on two calls in a row
where the second is smaller, for the bf16 MFMA decode path, the bf16 and
W8A8 row-streaming paths and the 4-bit path; sizes beyond the static scratch
are refused before anything is enqueued."""
import gc

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


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def case(cfg, T, S, seed):
    li = synth.LayerInputs(cfg, T=T, step=seed)
    z = oracle.logits(li.x, li.x_dtype, li.G)
    ids = oracle.topk(z, li.k)
    w = oracle.route_weights(z, ids)
    rng = np.random.default_rng(seed)
    resident = rng.choice(li.E, S, replace=False)
    e2s = np.full(li.E, -1, np.int32)
    e2s[resident] = np.arange(S)
    sl = e2s[ids].astype(np.int32)
    x = dev(li.x.view(np.int16) if li.x_dtype else li.x)
    return li, x, dev(sl), dev(w), dev(li.store[resident]), S


def both(m, li, x, sl, w, slots, S):
    T, k, H, I = li.T, li.k, li.H, li.I
    ws_b = m.moe_ffn_workspace_bytes(T, k, S, li.w_type, H, I)
    assert ws_b <= m.moe_ffn_noalloc_scratch_bytes()
    ws = torch.empty(ws_b, dtype=torch.uint8, device="cuda")
    y_ref = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    m.moe_ffn_slots(x, li.x_dtype, sl, w, T, k, slots, li.slab, S, li.w_type, H, I, y_ref, ws, ws_b)
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    gc.collect()  # tensors of earlier cases are freed now, not during the call
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    m.moe_ffn_slots_noalloc(x, li.x_dtype, sl, w, T, k, slots, li.slab, S, li.w_type, H, I, y)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() <= before  # nothing allocated through torch by the call
    return y.cpu().numpy(), y_ref.cpu().numpy()


@pytest.mark.parametrize("cfg,T1,T2,S", [("c2", 64, 8, 64), ("c3", 16, 3, 32), ("c4", 32, 1, 192), ("c1", 16, 5, 4)])
def test_noalloc_equals_workspace_entry_two_calls(m, cfg, T1, T2, S):
    for i, T in enumerate((T1, T2)):  # the second call is smaller and reuses the scratch the first left behind
        li, x, sl, w, slots, S_ = case(cfg, T, S, 11 + i)
        y, y_ref = both(m, li, x, sl, w, slots, S_)
        assert not np.isnan(y).any()
        np.testing.assert_array_equal(y, y_ref, err_msg=f"{cfg} call {i + 1} (T={T})")


def test_noalloc_refuses_sizes_beyond_the_scratch(m):
    E, k, H, I, T = 288, 8, 4096, 1536, 2048
    assert m.moe_ffn_workspace_bytes(T, k, E, 1, H, I) > m.moe_ffn_noalloc_scratch_bytes()
    slab = synth.slab_bytes(1, H, I)
    x = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    sl = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    slots = torch.zeros(16, dtype=torch.uint8, device="cuda")
    y = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    with pytest.raises(m.MoeError) as e:
        m.moe_ffn_slots_noalloc(x, 1, sl, w, T, k, slots, slab, E, 1, H, I, y)
    assert e.value.code == m.MOE_E_SHAPE and "static scratch" in str(e.value)


@pytest.mark.parametrize("cfg,T,S,other", [("c2", 64, 64, 8), ("c2", 1, 64, 8), ("c3", 16, 32, 3), ("c4", 32, 192, 1)])
def test_noalloc_replayed_from_a_hip_graph(m, cfg, T, S, other):
    """The allocation-free call captured once in a HIP graph and replayed
    three times, with eager calls of another size on the same static scratch
    between the replays: every replay equals the eager result bit for bit (the
    kernels clear what they count in, so a replay does not depend on what the
    scratch held)."""
    li, x, sl, w, slots, S = case(cfg, T, S, seed=11)
    lo, xo, slo, wo, slotso, So = case(cfg, other, S, seed=12)
    _, y_ref = both(m, li, x, sl, w, slots, S)

    def call(L, xx, ss, ww, st, SS, out):
        m.moe_ffn_slots_noalloc(xx, L.x_dtype, ss, ww, L.T, L.k, st, L.slab, SS, L.w_type, L.H, L.I, out)

    y = torch.full((li.T, li.H), float("nan"), dtype=torch.float32, device="cuda")
    y_other = torch.empty((lo.T, lo.H), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(li, x, sl, w, slots, S, y)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(li, x, sl, w, slots, S, y)
    torch.cuda.synchronize()
    for rep in range(3):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy(), y_ref, err_msg=f"replay {rep}")
        call(lo, xo, slo, wo, slotso, So, y_other)  # eager work on the same scratch between replays
        torch.cuda.synchronize()
