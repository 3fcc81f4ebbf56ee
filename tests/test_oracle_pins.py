"""Pins of the CPU oracle to facts other than itself (no GPU needed).

Each test ties one oracle function to a closed form, a brute-force search, a
textbook algorithm written independently here, a numpy/scipy routine, or a
number the pages print (tests/golden/page_facts.json).  A plausible slip in
the oracle -- a dropped term, a wrong sign or index, a transposed operand,
a wrong tie-break -- fails at least one of them.
"""
import itertools
import json
import math
import os
from collections import OrderedDict

import numpy as np
import pytest
import scipy.special

import oracle
import synth

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))
rng = np.random.default_rng(1234)


def silu(v):
    return v / (1.0 + np.exp(-v))


# ------------------------------------------------------------------ formats


def test_bf16_decode_known_patterns():
    H, I = 32, 32
    pats = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x3F00, 0x4049, 0x7F7F, 0x0001], np.uint16)
    expect = np.array([1.0, -2.0, 0.0, -0.0, 0.5, 3.140625, 3.3895313892515355e38, 9.183549615799121e-41])
    slab = np.zeros(oracle.slab_bytes(1, H, I), np.uint8)
    slab[:16] = pats.view(np.uint8)
    wg, _, _ = oracle.decode_expert(1, slab, H, I)
    np.testing.assert_array_equal(wg.reshape(-1)[:8].astype(np.float64), expect.astype(np.float32).astype(np.float64))
    assert np.signbit(wg.reshape(-1)[3])


def test_fp16_scales_match_numpy_float16():
    """4-bit scales decode as IEEE binary16 (numpy's float16 is the reference)."""
    H, I = 32, 32
    slab = np.zeros(oracle.slab_bytes(3, H, I), np.uint8)
    nib_plane = H * I // 2
    halves = np.array([0x3C00, 0x3800, 0x0001, 0x7BFF, 0x8400, 0x03FF, 0x4248, 0xC500], np.uint16)
    # gate rows 0..7, block 0: scale halves[r]; all codes 9 -> value = scale * (9 - 8)
    for r in range(8):
        slab[r * (H // 2):(r + 1) * (H // 2)] = 0x99
        slab[nib_plane + 2 * r * (H // 32):nib_plane + 2 * r * (H // 32) + 2] = np.frombuffer(
            halves[r:r + 1].tobytes(), np.uint8)
    wg, _, _ = oracle.decode_expert(3, slab, H, I)
    ref = halves.view(np.float16).astype(np.float32)
    for r in range(8):
        np.testing.assert_array_equal(wg[r], np.full(H, ref[r], np.float32))


def test_q4_nibble_order_and_offset():
    """Byte j of a block holds input j (low nibble) and input j+16 (high)."""
    H, I = 64, 32
    slab = np.zeros(oracle.slab_bytes(3, H, I), np.uint8)
    codes = rng.integers(0, 16, size=(I, H))
    for r in range(I):
        for b in range(H // 32):
            blk = codes[r, 32 * b:32 * b + 32]
            slab[r * (H // 2) + 16 * b:r * (H // 2) + 16 * b + 16] = (blk[:16] | (blk[16:] << 4)).astype(np.uint8)
    sc_off = I * H // 2
    one = np.frombuffer(np.array([0x3C00], np.uint16).tobytes(), np.uint8)
    for r in range(I):
        for b in range(H // 32):
            o = sc_off + 2 * (r * (H // 32) + b)
            slab[o:o + 2] = one
    wg, _, _ = oracle.decode_expert(3, slab, H, I)
    np.testing.assert_array_equal(wg, (codes - 8).astype(np.float32))


@pytest.mark.parametrize("w_type", [0, 1, 2, 3])
def test_encode_decode_round_trip_error_bounds(w_type):
    H, I = 64, 96
    wg = rng.normal(0, 0.02, (I, H)).astype(np.float32)
    wu = rng.normal(0, 0.02, (I, H)).astype(np.float32)
    wd = rng.normal(0, 0.02, (H, I)).astype(np.float32)
    slab = synth.encode_slab(w_type, H, I, wg, wu, wd)
    assert slab.size == oracle.slab_bytes(w_type, H, I) == synth.slab_bytes(w_type, H, I)
    dg, du, dd = oracle.decode_expert(w_type, slab, H, I)
    for src, dec in ((wg, dg), (wu, du), (wd, dd)):
        err = np.abs(dec.astype(np.float64) - src)
        if w_type == 0:
            assert err.max() == 0
        elif w_type == 1:
            assert np.all(err <= np.abs(src) * 2.0 ** -8)
        elif w_type == 2:
            s = np.abs(src).max(axis=1, keepdims=True) / 127
            assert np.all(err <= s * 0.5 * (1 + 1e-6))
        else:
            blocks = np.abs(src).reshape(src.shape[0], -1, 32).max(axis=2) / 7
            bound = np.repeat(blocks, 32, axis=1) * (0.5 + 2e-3)
            assert np.all(err <= bound + 1e-12)


def test_slab_sizes_match_page_numbers():
    # per-expert slab sizes of the five workloads
    assert oracle.slab_bytes(0, 64, 128) == 98_304
    assert oracle.slab_bytes(1, 2048, 768) == 9_437_184
    assert oracle.slab_bytes(2, 2048, 768) == 4_732_928
    assert oracle.slab_bytes(3, 2048, 512) == 1_769_472
    assert oracle.slab_bytes(1, 4096, 1536) == 37_748_736
    for t, h, i in [(0, 64, 128), (1, 2048, 768), (2, 2048, 768), (3, 2048, 512), (1, 4096, 1536)]:
        assert oracle.slab_bytes(t, h, i) % 16 == 0
    # 48 x 512 experts of 4-bit blocks: "~43 GB" held in host memory
    total = 48 * 512 * oracle.slab_bytes(3, 2048, 512)
    assert abs(total / 1e9 - GOLDEN["q4_stack_total"]["approx_gb"]) < 1.0
    # W8A8 expert over 48 layers: the sizing section's "~212 MB" per expert, "~27 GB" for 128
    per_expert = 48 * oracle.slab_bytes(2, 2048, 768)
    assert abs(per_expert / 2 ** 20 - GOLDEN["w8a8_expert_sizing"]["approx_mb_per_expert_all_layers"]) < 10
    assert abs(128 * per_expert / 2 ** 30 - GOLDEN["w8a8_expert_sizing"]["approx_gb_all_experts"]) < 1.0
    # bias table: 48 x 512 fp32 = "about 98 KB"
    assert 48 * 512 * 4 == 98_304
    assert abs(48 * 512 * 4 - GOLDEN["bias_table"]["approx_bytes"]) < 1000


# ------------------------------------------------------------------ router


def test_logits_exact_on_small_integers():
    T, H, E = 5, 48, 7
    x = rng.integers(-3, 4, size=(T, H)).astype(np.float32)
    G = rng.integers(-3, 4, size=(E, H)).astype(np.float32)
    z = oracle.logits(x, 0, G)
    np.testing.assert_array_equal(z, (x.astype(np.int64) @ G.astype(np.int64).T).astype(np.float32))


def test_logits_bf16_against_numpy_float64():
    li = synth.LayerInputs("c2", T=6, with_store=False)
    z = oracle.logits(li.x, 1, li.G)
    ref = (li.x_f32().astype(np.float64) @ li.G_f32().astype(np.float64).T).astype(np.float32)
    ulp = np.spacing(np.abs(ref))
    diff = np.abs(z - ref)
    assert np.all(diff <= ulp)
    assert np.mean(diff == 0) > 0.99


def _order_key(s, e):
    return (-s, e)


def test_topk_brute_force_all_subsets():
    """Every C(8,2) subset of a c1-shaped router: the pick is the unique set
    whose every member outranks every non-member under (score desc, id asc)."""
    li = synth.LayerInputs("c1", with_store=False)
    z = oracle.logits(li.x, 0, li.G)
    for k in (1, 2, 3):
        ids = oracle.topk(z, k)
        for t in range(z.shape[0]):
            good = []
            for sub in itertools.combinations(range(8), k):
                rest = [e for e in range(8) if e not in sub]
                if all(_order_key(z[t, a], a) < _order_key(z[t, b], b) for a in sub for b in rest):
                    good.append(sub)
            assert len(good) == 1
            assert sorted(ids[t]) == list(good[0])
            assert list(ids[t]) == sorted(good[0], key=lambda e: _order_key(z[t, e], e))


def test_topk_ties_go_to_lower_id_and_match_lexsort():
    z = np.array([[1.0, 3.0, 3.0, 2.0, 3.0, -1.0]], np.float32)
    assert list(oracle.topk(z, 3)[0]) == [1, 2, 4]
    assert list(oracle.topk(z, 4)[0]) == [1, 2, 4, 3]
    zz = np.round(rng.normal(0, 2, (64, 512)) * 4).astype(np.float32) / 4  # many exact ties
    ids = oracle.topk(zz, 10)
    for t in range(64):
        order = np.lexsort((np.arange(512), -zz[t].astype(np.float64)))
        assert list(ids[t]) == list(order[:10])


def test_topk_bias_none_is_bit_for_bit_unchanged():
    """'Nudge, don't cut' / 'The method in five lines': opt-in; unset changes nothing."""
    z = rng.normal(0, 2.3, (32, 512)).astype(np.float32)
    a = oracle.topk(z, 10)
    b = oracle.topk(z, 10, bias=np.zeros(512, np.float32))
    np.testing.assert_array_equal(a, b)


def test_topk_biased_score_is_one_fp32_add():
    z = rng.normal(0, 2.3, (32, 512)).astype(np.float32)
    bias = -rng.uniform(0, 1, 512).astype(np.float32)
    ids = oracle.topk(z, 10, bias)
    s = z + bias  # numpy float32 add
    for t in range(32):
        order = np.lexsort((np.arange(512), -s[t].astype(np.float64)))
        assert list(ids[t]) == list(order[:10])


def test_route_weights_sum_to_one_and_logistic_closed_form():
    z = rng.normal(0, 2.3, (200, 128)).astype(np.float32)
    for k in (1, 2, 8):
        ids = oracle.topk(z, k)
        w = oracle.route_weights(z, ids)
        assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= k * 2.0 ** -24)
        if k == 1:
            assert np.all(w == 1.0)
        if k == 2:
            z0 = z[np.arange(200), ids[:, 0]].astype(np.float64)
            z1 = z[np.arange(200), ids[:, 1]].astype(np.float64)
            ref = 1.0 / (1.0 + np.exp(z1 - z0))
            np.testing.assert_allclose(w[:, 0], ref, rtol=2 ** -23)
            np.testing.assert_allclose(w[:, 1], 1 - ref, rtol=2 ** -22)


def test_route_weights_use_raw_logits_not_biased_scores():
    """Selection only: the bias changes which experts run, not their weights."""
    z = rng.normal(0, 2.3, (50, 512)).astype(np.float32)
    bias = np.where(rng.uniform(size=512) < 0.6, -1.0, 0.0).astype(np.float32)
    ids = oracle.topk(z, 10, bias)
    w = oracle.route_weights(z, ids)
    for t in range(50):
        ref = scipy.special.softmax(z[t, ids[t]].astype(np.float64))
        np.testing.assert_allclose(w[t], ref, rtol=1e-6)
    # and the biased selection does differ from the unbiased one somewhere
    assert np.any(oracle.topk(z, 10) != ids)


def test_route_weights_shift_invariant():
    z = rng.normal(0, 2.3, (40, 64)).astype(np.float32)
    ids = oracle.topk(z, 4)
    w1 = oracle.route_weights(z, ids)
    w2 = oracle.route_weights(z + np.float32(16.0), ids)
    np.testing.assert_allclose(w1, w2, rtol=2e-6)


# -------------------------------------------------------------------- bias


def test_bias_table_edge_tail_cap_and_hot():
    E, n_hot, cap = 512, 192, -1.0
    b = synth.dirichlet(synth.key(7, synth.TAG_B), E, 0.3)
    bias = oracle.bias_table(b, n_hot, cap)
    order = np.lexsort((np.arange(E), -b))
    hot, cold = order[:n_hot], order[n_hot:]
    assert np.all(bias[hot] == 0.0)
    b_edge = b[order[n_hot - 1]]
    for e in cold:
        if b[e] <= b_edge * math.exp(cap):
            assert bias[e] == np.float32(cap)
        else:
            assert cap < bias[e] <= 0.0
            assert abs(bias[e] - math.log(b[e] / b_edge)) <= 1e-6
    # monotone: brighter cold experts never get a larger penalty
    cb = bias[cold]
    assert np.all(np.diff(cb) <= 0)
    assert bias.nbytes * 48 == 98_304


def test_bias_flat_hot_set_value_and_hard_mask():
    """'Nudge, don't cut' / 'Experts that don't fit': the hot set is kept at 0,
    every other expert gets one flat number; -inf is the hard mask, under
    which the picks are the plain top-k of the hot experts alone."""
    E, n_hot, k = 512, 192, 10
    b = synth.dirichlet(synth.key(11, synth.TAG_B), E, 0.3)
    order = np.lexsort((np.arange(E), -b))
    hot = np.sort(order[:n_hot])
    for v in (-0.5, -0.75, -1.0):
        bias = oracle.bias_flat(b, n_hot, v)
        assert np.all(bias[hot] == 0.0)
        assert np.sum(bias == np.float32(v)) == E - n_hot
        # the same hot set as the graded table (its zeros)
        np.testing.assert_array_equal(np.flatnonzero(oracle.bias_table(b, n_hot, -1.0) == 0.0), hot)
    mask = oracle.bias_flat(b, n_hot, -np.inf)
    z = rng.normal(0, 2.3, (40, E)).astype(np.float32)
    ids = oracle.topk(z, k, mask)
    for t in range(40):
        sub = np.lexsort((hot, -z[t, hot].astype(np.float64)))
        assert list(ids[t]) == list(hot[sub[:k]])
    # value 0 is no bias at all, bit for bit
    np.testing.assert_array_equal(oracle.topk(z, k, oracle.bias_flat(b, n_hot, 0.0)), oracle.topk(z, k))


def test_bias_affinity_values_zero_lambda_and_monotone_hits():
    """'Then Maya's own knob beat ours': lambda is added to the score of every
    expert resident now.  lambda = 0 changes nothing; a larger lambda never
    lowers the number of resident picks of a token; a lambda above the logit
    range makes the picks the top-k of the resident experts alone."""
    E, S, k = 128, 32, 8
    e2s = np.full(E, -1, np.int32)
    res = np.sort(rng.choice(E, S, replace=False))
    e2s[res] = np.arange(S)
    base = -rng.uniform(0, 1, E).astype(np.float32)
    a = oracle.bias_affinity(e2s, 0.25)
    assert np.all(a[res] == np.float32(0.25)) and np.sum(a == 0.0) == E - S
    np.testing.assert_array_equal(oracle.bias_affinity(e2s, 0.0, base), base)
    ab = oracle.bias_affinity(e2s, 0.25, base)
    ref = base.copy()
    ref[res] = base[res] + np.float32(0.25)  # one fp32 add
    np.testing.assert_array_equal(ab, ref)
    z = rng.normal(0, 2.3, (200, E)).astype(np.float32)
    prev = None
    for lam in (0.0, 0.125, 0.25, 0.5, 1.0, 2.0):
        ids = oracle.topk(z, k, oracle.bias_affinity(e2s, lam))
        hits = (e2s[ids] >= 0).sum(1)
        if prev is not None:
            assert np.all(hits >= prev)
        prev = hits
    big = np.float32(2.0 * (z.max() - z.min()) + 1.0)
    ids = oracle.topk(z, k, oracle.bias_affinity(e2s, big))
    for t in range(200):
        assert np.all(e2s[ids[t]] >= 0)
        sub = np.lexsort((res, -(z[t, res] + big).astype(np.float64)))
        assert list(ids[t]) == list(res[sub[:k]])


def test_route_weights_damped_closed_form():
    """'Qwen on Strata': damped weights are the softmax of the biased scores
    fl32(z + bias); with no bias (or one bias for all picks) they are the
    selection-only weights."""
    E = 256
    z = rng.normal(0, 2.3, (100, E)).astype(np.float32)
    bias = np.where(rng.uniform(size=E) < 0.5, -0.75, 0.0).astype(np.float32)
    ids2 = oracle.topk(z, 2, bias)
    w = oracle.route_weights_damped(z, bias, ids2)
    s = (z + bias).astype(np.float32)
    s0 = s[np.arange(100), ids2[:, 0]].astype(np.float64)
    s1 = s[np.arange(100), ids2[:, 1]].astype(np.float64)
    np.testing.assert_allclose(w[:, 0], 1.0 / (1.0 + np.exp(s1 - s0)), rtol=2 ** -23)
    ids = oracle.topk(z, 8, bias)
    wd = oracle.route_weights_damped(z, bias, ids)
    assert np.all(np.abs(wd.astype(np.float64).sum(1) - 1.0) <= 8 * 2.0 ** -24)
    np.testing.assert_array_equal(oracle.route_weights_damped(z, None, ids), oracle.route_weights(z, ids))
    same = np.full(E, -0.75, np.float32)  # one shift for every pick: the softmax does not move
    np.testing.assert_allclose(oracle.route_weights_damped(z, same, ids), oracle.route_weights(z, ids), rtol=2e-6)
    # a pick that carries the penalty weighs less than it would selection-only
    ws = oracle.route_weights(z, ids)
    pen = bias[ids] < 0
    mixed = pen.any(1) & ~pen.all(1)
    assert np.all(wd[mixed][pen[mixed]] < ws[mixed][pen[mixed]])


def test_bias_table_hand_values():
    # b_edge = 0.2 (weakest of the two hot experts)
    b = np.array([0.4, 0.2, 0.2, 0.2 * math.exp(-0.5), 0.2 * math.exp(-3), 0.0])
    bias = oracle.bias_table(b, 2, -1.0)
    assert bias[0] == 0 and bias[1] == 0
    assert bias[2] == 0.0  # same brightness as the edge: ln 1
    assert abs(bias[3] - (-0.5)) <= 2 ** -24
    assert bias[4] == np.float32(-1.0)  # deep tail -> cap
    assert bias[5] == np.float32(-1.0)  # b = 0 -> cap
    assert np.all(oracle.bias_table(b, 6, -1.0) == 0)


# ---------------------------------------------------------- cache manager


class TextbookLRU:
    def __init__(self, S):
        self.slots = [None] * S
        self.order = OrderedDict()

    def access(self, e):
        if e in self.order:
            self.order.move_to_end(e)
            return True, None
        if None in self.slots:
            s = self.slots.index(None)
        else:
            victim = next(iter(self.order))
            del self.order[victim]
            s = self.slots.index(victim)
        self.slots[s] = e
        self.order[e] = True
        return False, s


class TextbookLFU:
    def __init__(self, S):
        self.slots = [None] * S
        self.count = {}
        self.used = {}
        self.clock = 0

    def access(self, e):
        now = self.clock
        self.clock += 1
        if e in self.count:
            self.count[e] += 1
            self.used[e] = now
            return True, None
        if None in self.slots:
            s = self.slots.index(None)
        else:
            victim = min(self.count, key=lambda v: (self.count[v], self.used[v], self.slots.index(v)))
            del self.count[victim], self.used[victim]
            s = self.slots.index(victim)
        self.slots[s] = e
        self.count[e] = 1
        self.used[e] = now
        return False, s


@pytest.mark.parametrize("policy,Ref", [("lru", TextbookLRU), ("lfu", TextbookLFU)])
@pytest.mark.parametrize("S", [1, 3, 5])
@pytest.mark.parametrize("dist", ["uniform", "zipf"])
def test_manage_single_request_steps_are_textbook(policy, Ref, S, dist):
    E, n = 12, 400
    if dist == "uniform":
        seq = rng.integers(0, E, n)
    else:
        seq = synth.zipf_ids(synth.key(3, 7), synth.key(3, 8, S), n, E, 1, 0.8).reshape(-1)
    c = oracle.Cache(E, S, policy)
    ref = Ref(S)
    for e in seq:
        r = c.manage(np.array([e]))
        hit, slot = ref.access(int(e))
        assert (r["stats"][0] == 1) == hit
        if hit:
            assert r["miss"].shape[0] == 0
        else:
            assert r["miss"].tolist() == [[int(e), slot]]
        assert r["slot_ids"][0] == (c.e2s[e])
        assert [None if v < 0 else int(v) for v in c.s2e] == ref.slots
        if policy == "lfu":
            # priorities themselves: use count since insertion, step of last use
            for s_, e_ in enumerate(ref.slots):
                if e_ is not None:
                    assert c.freq[s_] == ref.count[e_] and c.last[s_] == ref.used[e_]


def _check_manage_invariants(c, before_e2s, ids, r, policy, S):
    E = c.E
    ids = ids.reshape(-1)
    need = sorted(set(ids.tolist()))
    # maps are mutual inverses
    for s in range(S):
        if c.s2e[s] >= 0:
            assert c.e2s[c.s2e[s]] == s
    for e in range(E):
        if c.e2s[e] >= 0:
            assert c.s2e[c.e2s[e]] == e
    resident = {e for e in range(E) if c.e2s[e] >= 0}
    host = r["host_miss"].tolist()
    assert set(need) <= resident | set(host)
    assert not (set(host) & resident)
    assert host == sorted(host) and len(set(host)) == len(host)
    miss = r["miss"]
    assert miss[:, 0].tolist() == sorted(miss[:, 0].tolist())
    assert len(set(miss[:, 1].tolist())) == len(miss)
    # the gathered experts were not resident before; the victims held nothing needed
    for e, s in miss.tolist():
        assert before_e2s[e] < 0
    st = r["stats"]
    assert st[0] == sum(1 for e in ids if before_e2s[e] >= 0)
    assert st[1] == len(need)
    assert st[2] == len(miss) and st[3] == len(host)
    assert len(need) == sum(1 for e in need if before_e2s[e] >= 0) + st[2] + st[3]
    np.testing.assert_array_equal(r["slot_ids"], c.e2s[ids])


@pytest.mark.parametrize("policy", ["lru", "lfu", "static"])
def test_manage_invariants_multi_id_steps(policy):
    E, S, T, k = 128, 32, 16, 8
    resident = list(range(0, 2 * S, 2)) if policy == "static" else None
    c = oracle.Cache(E, S, policy, resident=resident)
    kp, kd = synth.key(5, 7), synth.key(5, 8)
    all_ids = synth.zipf_ids(kp, kd, 40 * T, E, k, 0.8).reshape(40, T, k)
    for step in range(40):
        before = c.e2s.copy(), c.s2e.copy(), c.last.copy(), c.freq.copy()
        r = c.manage(all_ids[step])
        _check_manage_invariants(c, before[0], all_ids[step], r, policy, S)
        need = set(all_ids[step].reshape(-1).tolist())
        if policy == "static":
            np.testing.assert_array_equal(c.e2s, before[0])
            np.testing.assert_array_equal(c.s2e, before[1])
            assert r["miss"].shape[0] == 0
        else:
            # victims are the first candidates in (empty first, then policy key, then slot) order
            b_e2s, b_s2e, b_last, b_freq = before
            cand = [s for s in range(S) if b_s2e[s] < 0 or b_s2e[s] not in need]
            hits_last = b_last.copy()
            hits_freq = b_freq.copy()
            for e in need:
                if b_e2s[e] >= 0:
                    hits_last[b_e2s[e]] = step
                    hits_freq[b_e2s[e]] += 1
            if policy == "lru":
                keyf = lambda s: (b_s2e[s] >= 0, hits_last[s] if b_s2e[s] >= 0 else 0, s)
            else:
                keyf = lambda s: (b_s2e[s] >= 0, hits_freq[s] if b_s2e[s] >= 0 else 0,
                                  hits_last[s] if b_s2e[s] >= 0 else 0, s)
            cand.sort(key=keyf)
            assert r["miss"][:, 1].tolist() == cand[:len(r["miss"])]
            assert c.step[0] == step + 1


def test_manage_sizing_trap_rule():
    """'Measuring, without fooling yourself': tokens x top_k <= slots means the
    step is served from slots alone (no host misses) under a dynamic policy."""
    trap = GOLDEN["sizing_trap"]
    E = 128
    for S in (trap["example_ids"], trap["example_ids"] + 8):
        c = oracle.Cache(E, S, "lru")
        ids = synth.zipf_ids(synth.key(9, 7), synth.key(9, 8, S), 50 * trap["example_tokens"], E,
                             trap["example_top_k"], 0.8).reshape(50, -1)
        for step in range(50):
            r = c.manage(ids[step])
            assert r["stats"][3] == 0
    # one slot short: some step must overflow to the host pass
    c = oracle.Cache(E, trap["example_ids"] - 1, "lru")
    overflow = 0
    ids = np.stack([rng.permutation(E)[:trap["example_ids"]] for _ in range(50)]).astype(np.int32)
    for step in range(50):
        overflow += c.manage(ids[step])["stats"][3] > 0
    assert overflow > 0


def test_manage_deterministic():
    ids = synth.zipf_ids(synth.key(11, 7), synth.key(11, 8), 30 * 16, 128, 8, 0.8).reshape(30, -1)
    outs = []
    for _ in range(2):
        c = oracle.Cache(128, 32, "lfu")
        outs.append([c.manage(ids[s]) for s in range(30)])
    for a, b in zip(*outs):
        for key in a:
            np.testing.assert_array_equal(a[key], b[key])


def test_repick_swaps_only_what_went_cold():
    """[RTX] 'Full Transcript': every ~500 tokens have another look, swap out
    whatever has gone cold and leave the rest alone.  Written independently:
    the set after a repick is the new set; members already resident keep
    their slots; exactly the new members are loaded, in ascending id, into the
    freed slots in ascending order; a second repick to the same set loads
    nothing."""
    r = np.random.default_rng(77)
    for _ in range(50):
        E = int(r.integers(4, 40))
        S = int(r.integers(1, E + 1))
        old = r.choice(E, S, replace=False)
        new = r.choice(E, S, replace=False)
        c = oracle.Cache(E, S, "static", resident=old)
        c.last[:] = r.integers(1, 1000, S)
        c.freq[:] = r.integers(1, 1000, S)
        c.step[0] = 4321
        slots_before, last_before, freq_before = c.e2s.copy(), c.last.copy(), c.freq.copy()
        loads = c.repick(new)
        # a loaded slot restarts (last = the current step, no uses); a kept slot keeps its record;
        # a repick is not a step
        ls = loads[:, 1]
        assert np.all(c.last[ls] == 4321) and np.all(c.freq[ls] == 0) and c.step[0] == 4321
        keep = np.setdiff1d(np.arange(S), ls)
        assert np.array_equal(c.last[keep], last_before[keep]) and np.array_equal(c.freq[keep], freq_before[keep])
        assert set(np.flatnonzero(c.e2s >= 0)) == set(new.tolist())
        assert sorted(c.s2e.tolist()) == sorted(new.tolist())
        assert np.all(c.e2s[c.s2e] == np.arange(S))
        kept = set(old.tolist()) & set(new.tolist())
        for e in kept:
            assert c.e2s[e] == slots_before[e]
        loaded = sorted(set(new.tolist()) - set(old.tolist()))
        assert loads[:, 0].tolist() == loaded
        freed = sorted(slots_before[e] for e in set(old.tolist()) - set(new.tolist()))
        assert loads[:, 1].tolist() == freed
        assert len(c.repick(c.s2e.copy())) == 0
    # a repeated or out-of-range entry is skipped; an unneeded slot keeps its expert
    c = oracle.Cache(10, 4, "static", resident=[1, 2, 3, 4])
    loads = c.repick(np.array([3, 7, 7, 42], np.int32))
    assert loads.tolist() == [[7, 0]]
    assert c.s2e.tolist() == [7, 2, 3, 4]
    # from an empty cache the new set fills slots 0.. in ascending id
    c = oracle.Cache(10, 3, "static")
    assert c.repick(np.array([9, 2, 5], np.int32)).tolist() == [[2, 0], [5, 1], [9, 2]]


def test_best_fixed_set_is_the_most_picked():
    """The perfect-foresight fixed set of [RTX] 'Full Transcript' (see the
    whole run, pick the best fixed set before starting): over every subset of
    S experts, none serves more routing ids of the trace than the S most
    picked (pick_static over the whole trace)."""
    r = np.random.default_rng(5)
    E, S = 9, 3
    for _ in range(10):
        trace = r.choice(E, 200, p=r.dirichlet(np.ones(E) * 0.5)).astype(np.int32)
        counts = np.bincount(trace, minlength=E)
        best = max(counts[list(sub)].sum() for sub in itertools.combinations(range(E), S))
        assert counts[oracle.pick_static(trace, E, S)].sum() == best


def test_gather_bytes_equal_source_rows():
    E, S, sb = 10, 4, 96
    host = rng.integers(0, 256, (E, sb)).astype(np.uint8)
    slots = np.zeros((S, sb), np.uint8)
    miss = np.array([[7, 2], [1, 0], [9, 3]], np.int32)
    oracle.gather(miss, host, slots)
    for e, s in miss:
        assert bytes(slots[s]) == bytes(host[e])
    assert not slots[1].any()


def test_pick_static_counts():
    ids = np.array([[3, 1], [3, 2], [1, 3], [0, 5], [5, 3]], np.int32)
    assert oracle.pick_static(ids, 6, 3).tolist() == [3, 1, 5]
    assert oracle.pick_static(ids, 6, 6).tolist() == [3, 1, 5, 0, 2, 4]


# -------------------------------------------------------------- expert FFN


def _dense_swiglu(wg, wu, wd, x, h_round=None):
    g = wg.astype(np.float64) @ x
    u = wu.astype(np.float64) @ x
    h = silu(g) * u
    if h_round is not None:
        h = h_round(h)
    return wd.astype(np.float64) @ h


def _bf16_round(h):
    return synth.bf16_to_f32(synth.f32_to_bf16(h.astype(np.float32))).astype(np.float64)


@pytest.mark.parametrize("w_type", [0, 1, 3])
def test_expert_equals_dense_swiglu(w_type):
    """k = 1, w = 1, one token: the layer is a plain dense SwiGLU MLP."""
    H, I = 64, 128
    x_dtype = 0 if w_type == 0 else 1
    slab = synth.slabs(w_type, 77, 0, 0, 1, H, I, 0.05)[0]
    x = synth.normal(synth.key(77, 1), (1, H), 1.0, x_dtype)
    xf = x.astype(np.float64) if x_dtype == 0 else synth.bf16_to_f32(x).astype(np.float64)
    wg, wu, wd = oracle.decode_expert(w_type, slab, H, I)
    ref = _dense_swiglu(wg, wu, wd, xf[0], None if w_type == 0 else _bf16_round)
    o = oracle.expert(w_type, slab, H, I, x[0], x_dtype)
    np.testing.assert_allclose(o, ref, rtol=1e-9, atol=1e-12)
    # and through the layer with k = 1, w = 1
    store = slab[None, :]
    yf, _, _ = oracle.layer(w_type, store, 1, H, I, x, x_dtype, np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32))
    np.testing.assert_allclose(yf[0], ref.astype(np.float32), rtol=1e-6, atol=1e-9)


def test_expert_w8a8_close_to_dequantised_dense():
    """W8A8 differs from the float layer only by int8 rounding of x and h."""
    H, I = 256, 128
    slab = synth.slabs(2, 78, 0, 0, 1, H, I, 0.05)[0]
    x = synth.normal(synth.key(78, 1), (4, H), 1.0, 1)
    wg, wu, wd = oracle.decode_expert(2, slab, H, I)
    for t in range(4):
        xf = synth.bf16_to_f32(x[t]).astype(np.float64)
        ref = _dense_swiglu(wg, wu, wd, xf)
        o = oracle.expert(2, slab, H, I, x[t], 1)
        rms = np.sqrt(np.mean(ref ** 2))
        assert np.max(np.abs(o - ref)) <= 0.03 * rms + 0.03 * np.abs(ref).max()
        assert np.sqrt(np.mean((o - ref) ** 2)) <= 0.02 * rms


def _w8a8_hand_slab():
    """A 4 x 4 W8A8 expert whose every intermediate value is an exact integer.

    Gate codes pick x's second element with large multipliers, so every gate
    pre-activation is >= 41 and silu(g) == g exactly in double (e^-41 is below
    half an ulp of 1).  Scales: gate 1, up (0.5, 1, 1, 1), down (0.5, 1, 2,
    0.25) -- distinct, so a plane or index mix-up changes the result."""
    H = I = 4
    wg = np.array([[1, 0, 0, 0], [0, 41, 0, 0], [0, 43, 0, 0], [0, 45, 0, 0]], np.int8)
    wu = np.array([[0, 4, 0, 0], [0, 1, 0, 0], [0, 1, 0, 2], [0, -1, 7, 0]], np.int8)
    wd = np.array([[1, 0, 0, 0], [0, 1, 1, 0], [0, 0, 1, 1], [-1, 2, -3, 5]], np.int8)
    sg = np.array([1, 1, 1, 1], np.float32)
    su = np.array([0.5, 1, 1, 1], np.float32)
    sd = np.array([0.5, 1, 2, 0.25], np.float32)
    slab = np.concatenate([wg.reshape(-1).view(np.uint8), wu.reshape(-1).view(np.uint8),
                           wd.reshape(-1).view(np.uint8), sg.view(np.uint8), su.view(np.uint8), sd.view(np.uint8)])
    assert slab.size == oracle.slab_bytes(2, H, I)
    return slab, H, I


def test_expert_w8a8_exact_hand_derived():
    """W8A8 arithmetic pinned to values worked out by hand (BASELINE config 3:
    int8 weights with per-output-channel fp32 scales, per-token int8
    activations; reading: scale absmax/127, round half to even, clamp 127,
    h requantised per (token, pick) row).

    token 0: x = (127, 1, 0, 0): absmax 127 -> s_x = 1, codes = x.
      g = (127, 41, 43, 45); u = (4*0.5, 1, 1, -1) = (2, 1, 1, -1)
      h = g*u = (254, 41, 43, -45); s_h = 254/127 = 2
      h/s_h = (127, 20.5, 21.5, -22.5) -> half to even (127, 20, 22, -22)
      down acc = (127, 20+22, 22-22, -127+40-66-110) = (127, 42, 0, -263)
      o = acc * 2 * (0.5, 1, 2, 0.25) = (127, 84, 0, -131.5)
    token 1: x = (254, 2, 1, 3): absmax 254 -> s_x = 2,
      x/s_x = (127, 1, 0.5, 1.5) -> codes (127, 1, 0, 2)
      g = 2*(127, 41, 43, 45) = (254, 82, 86, 90)
      u acc = (4, 1, 1+2*2, -1+7*0) = (4, 1, 5, -1); u = acc*2*s_u = (4, 2, 10, -2)
      h = (1016, 164, 860, -180); s_h = 1016/127 = 8
      h/s_h = (127, 20.5, 107.5, -22.5) -> (127, 20, 108, -22)
      down acc = (127, 128, 86, -127+40-324-110) = (127, 128, 86, -521)
      o = acc * 8 * s_d = (508, 1024, 1376, -1042)
    A truncating quantiser (21.5 -> 21), half away from zero (20.5 -> 21),
    a /128 scale, a per-tensor activation scale (token 0 would get s_x = 2
    and codes 63.5 -> 64) or an h scale shared by the tokens each change at
    least one of these outputs."""
    slab, H, I = _w8a8_hand_slab()
    x = synth.f32_to_bf16(np.array([[127, 1, 0, 0], [254, 2, 1, 3]], np.float32))
    want = np.array([[127, 84, 0, -131.5], [508, 1024, 1376, -1042]], np.float64)
    for t in range(2):
        o = oracle.expert(2, slab, H, I, x[t], 1)
        assert np.array_equal(o, want[t]), (t, o, want[t])
    # the same through the layer: one expert, k = 1, w = 1, both tokens in one call
    yf, yg, yh = oracle.layer(2, slab[None, :], 1, H, I, x, 1, np.zeros((2, 1), np.int32),
                              np.ones((2, 1), np.float32), slot_ids=np.zeros((2, 1), np.int32))
    assert np.array_equal(yf, want.astype(np.float32))
    assert np.array_equal(yg, want.astype(np.float32)) and np.all(yh == 0)


def test_expert_w8a8_zero_row_takes_scale_one():
    """An all-zero activation row takes scale 1 (codes 0): the output is +0,
    not NaN from 0/0."""
    slab, H, I = _w8a8_hand_slab()
    o = oracle.expert(2, slab, H, I, np.zeros(H, np.uint16), 1)
    assert np.all(o == 0) and not np.any(np.signbit(o))


@pytest.mark.parametrize("w_type", [0, 1, 2, 3])
def test_expert_zero_input_gives_zero(w_type):
    H, I = 64, 64
    slab = synth.slabs(w_type, 79, 0, 0, 1, H, I, 0.02)[0]
    x = np.zeros(H, np.float32 if w_type == 0 else np.uint16)
    o = oracle.expert(w_type, slab, H, I, x, 0 if w_type == 0 else 1)
    assert np.all(o == 0)


def test_q4_all_codes_eight_gives_zero():
    H, I = 64, 64
    slab = synth.slabs(3, 80, 0, 0, 1, H, I, 0.02)[0].copy()
    n = H * I
    for p in range(3):
        base = p * (n // 2 + n // 16)
        slab[base:base + n // 2] = 0x88
    x = synth.normal(synth.key(80, 1), (H,), 1.0, 1)
    assert np.all(oracle.expert(3, slab, H, I, x, 1) == 0)


def test_layer_is_linear_in_routing_weights():
    li = synth.LayerInputs("c1")
    z = oracle.logits(li.x, 0, li.G)
    ids = oracle.topk(z, 2)
    w = oracle.route_weights(z, ids)
    y1, _, _ = oracle.layer(0, li.store, 8, 64, 128, li.x, 0, ids, w)
    y2, _, _ = oracle.layer(0, li.store, 8, 64, 128, li.x, 0, ids, w * np.float32(0.5))
    np.testing.assert_allclose(y2, y1 * 0.5, rtol=1e-6, atol=1e-12)


# ------------------------------------------------------- cache equivalence


@pytest.mark.parametrize("cfg,T", [("c1", 16), ("c2", 4)])
def test_split_passes_sum_to_full_layer(cfg, T):
    """'What the video covers' / transcript: missing experts return zero, the
    two passes are summed, and the result is the layer without a cache."""
    li = synth.LayerInputs(cfg, T=T)
    E, H, I, k = li.E, li.H, li.I, li.k
    z = oracle.logits(li.x, li.x_dtype, li.G)
    ids = oracle.topk(z, k)
    w = oracle.route_weights(z, ids)
    S = {"c1": 4, "c2": 64}[cfg]
    resident = list(range(S)) if cfg == "c1" else oracle.pick_static(ids, E, S)
    c = oracle.Cache(E, S, "static", resident=resident)
    r = c.manage(ids)
    sl = r["slot_ids"].reshape(T, k)
    yf, yg, yh = oracle.layer(li.w_type, li.store, E, H, I, li.x, li.x_dtype, ids, w, sl)
    rms = np.sqrt(np.mean(yf.astype(np.float64) ** 2))
    assert np.max(np.abs((yg.astype(np.float64) + yh) - yf)) <= 1e-6 * rms
    # all resident (any slot permutation) == no cache, bit for bit
    perm = rng.permutation(E)
    _, yg_all, yh_all = oracle.layer(li.w_type, li.store, E, H, I, li.x, li.x_dtype, ids, w, perm[ids].astype(np.int32))
    np.testing.assert_array_equal(yg_all, yf)
    assert np.all(yh_all == 0)
    # nothing resident: the resident pass is exactly zero and the host pass is the layer
    _, yg0, yh0 = oracle.layer(li.w_type, li.store, E, H, I, li.x, li.x_dtype, ids, w, np.full_like(ids, -1))
    assert np.all(yg0 == 0) and not np.any(np.signbit(yg0))
    np.testing.assert_array_equal(yh0, yf)


def test_output_independent_of_slot_count():
    """Transcript: the output stays identical across the slot sweep."""
    li = synth.LayerInputs("c1")
    z = oracle.logits(li.x, 0, li.G)
    ids = oracle.topk(z, 2)
    w = oracle.route_weights(z, ids)
    sums = []
    for S in range(0, 9):
        c = oracle.Cache(8, S, "static", resident=list(range(S)))
        sl = c.manage(ids)["slot_ids"].reshape(ids.shape)
        yf, yg, yh = oracle.layer(0, li.store, 8, 64, 128, li.x, 0, ids, w, sl)
        sums.append(yg.astype(np.float64) + yh)
    for s in sums[1:]:
        np.testing.assert_allclose(s, sums[0], rtol=0, atol=1e-6 * np.abs(sums[0]).max())


# ------------------------------------------------------------- generator


def test_generator_deterministic_and_thread_independent(monkeypatch):
    a = synth.normal(synth.key(1, 2, 3, 4), (1000,), 1.0, 0)
    b = synth.normal(synth.key(1, 2, 3, 4), (1000,), 1.0, 0)
    np.testing.assert_array_equal(a, b)
    big = synth.normal(synth.key(5, 1), (300_000,), 0.02, 0)
    assert abs(big.mean()) < 0.02 * 0.01 and abs(big.std() / 0.02 - 1) < 0.01
    s1 = synth.slabs(1, 9, 0, 0, 4, 64, 128, 0.02)
    s2 = np.concatenate([synth.slabs(1, 9, 0, e, e + 1, 64, 128, 0.02) for e in range(4)])
    np.testing.assert_array_equal(s1, s2)


def test_generator_dirichlet_and_zipf():
    b = synth.dirichlet(synth.key(2, 6), 512, 0.3)
    assert abs(b.sum() - 1) < 1e-12 and np.all(b >= 0)
    ids = synth.zipf_ids(synth.key(2, 7), synth.key(2, 8), 4000, 128, 8, 0.8)
    assert all(len(set(r)) == 8 for r in ids)
    cnt = np.bincount(ids.reshape(-1), minlength=128)
    assert cnt.max() > 4 * max(cnt.min(), 1)


def test_residual_rounds_to_nearest_even_bf16():
    """Stack join x + y kept in bf16: exact sums stay, halfway cases go to the
    even neighbour, and fp32 streams add in fp32."""
    one = 0x3F80  # 1.0
    x = np.array([[one, one, one, one, 0xBF80, 0x0000]], np.uint16)
    # 1 + 2^-8 (exact bf16 step 2^-7 -> halfway, tie to even 1.0); 1 + 3*2^-8 (halfway, to 1 + 2^-6)
    # 1 + 2^-7 (exact); 1 + 0.75*2^-7 (rounds up); -1 + 1 = +0; 0 + 0 = 0
    y = np.array([[2.0 ** -8, 3 * 2.0 ** -8, 2.0 ** -7, 0.75 * 2.0 ** -7, 1.0, 0.0]], np.float32)
    got = oracle.residual(x, 1, y)
    want = [0x3F80, 0x3F82, 0x3F81, 0x3F81, 0x0000, 0x0000]
    assert got.reshape(-1).tolist() == want
    xf = np.array([[1.5, -2.25]], np.float32)
    np.testing.assert_array_equal(oracle.residual(xf, 0, np.array([[0.25, 0.25]], np.float32)), [[1.75, -2.0]])
