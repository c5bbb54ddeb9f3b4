"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against brute force on tiny inputs, an
independent dense formulation in torch, an invariance or a closed form, so a
plausible mistake in the oracle (dropped term, wrong index, transposed
operand, wrong sign, wrong order) fails at least one of them. The planted-
mistake tests at the end show that for several such mistakes.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_problem(seed, T=6, H=32, I=48, E=4, k=2, masked=0.0, dup=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    wg = (rng.standard_normal((E, I, H)) / math.sqrt(H)).astype(np.float32)
    wu = (rng.standard_normal((E, I, H)) / math.sqrt(H)).astype(np.float32)
    wd = (rng.standard_normal((E, H, I)) / math.sqrt(I)).astype(np.float32)
    if dup:
        ids = rng.integers(0, E, size=(T, k))
    else:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    if masked:
        ids = np.where(rng.random((T, k)) < masked, -1, ids)
    w = rng.random((T, k)).astype(np.float32)
    return x, ids.astype(np.int32), w, wg, wu, wd


# ------------------------------------------------------------------ align
def brute_align(ids, E):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    counts = [0] * E
    for v in flat:
        if 0 <= v < E:
            counts[v] += 1
    cu, run = [], 0
    for c in counts:
        run += c
        cu.append(run)
    perm = []
    for e in range(E):                     # segment by segment, slots in index order
        for i, v in enumerate(flat):
            if v == e:
                perm.append(i)
    inv = [-1] * len(flat)
    for p, i in enumerate(perm):
        inv[i] = p
    bad = sum(1 for v in flat if v != -1 and not (0 <= v < E))
    return counts, cu, perm, inv, bad


@pytest.mark.parametrize("seed", range(6))
def test_align_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    T, k, E = int(rng.integers(1, 40)), int(rng.integers(1, 5)), int(rng.integers(1, 9))
    ids = rng.integers(-1, E + 2, size=(T, k))         # includes masked (-1) and bad ids
    al = oracle.align(ids, E)
    counts, cu, perm, inv, bad = brute_align(ids, E)
    assert al["counts"].tolist() == counts
    assert al["cu_seqlens"].tolist() == cu
    assert al["offsets"].tolist() == [0] + cu
    assert al["perm"].tolist() == perm
    assert al["inv_perm"].tolist() == inv
    assert al["n_bad"] == bad


@pytest.mark.parametrize("name", ["tiny", "mixtral_prefill", "fine_grained_prefill", "mxfp4_decode"])
def test_align_invariants_on_workload_routing(name):
    wl = synth.workload(name)
    ids, _ = synth.make_routing(wl)
    al = oracle.align(ids, wl.E)
    flat = ids.reshape(-1)
    cu = al["cu_seqlens"]
    assert np.all(np.diff(np.concatenate([[0], cu])) >= 0)
    assert cu[-1] == flat.size                          # no masked ids in routed workloads
    assert sorted(al["perm"].tolist()) == list(range(flat.size))
    start = 0
    for e in range(wl.E):
        seg = al["perm"][start:cu[e]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)                 # stable: ascending slot index
        start = cu[e]
    assert np.all(al["inv_perm"][al["perm"]] == np.arange(flat.size))


# ------------------------------------------------------------------ grouped GEMM
def test_grouped_mm_matches_triple_loop():
    rng = np.random.default_rng(3)
    G, N, K = 4, 5, 7
    cu = [3, 3, 7, 9]                                   # segment 1 empty, rows 9..10 past the end
    a = rng.standard_normal((11, K))
    w = rng.standard_normal((G, N, K))
    got = oracle.grouped_mm(a, lambda g: w[g], cu)
    want = [[0.0] * N for _ in range(11)]
    start = 0
    for g, end in enumerate(cu):
        for r in range(start, end):
            for n in range(N):
                s = 0.0
                for kk in range(K):
                    s += a[r][kk] * w[g][n][kk]
                want[r][n] = s
        start = end
    np.testing.assert_allclose(got, np.array(want), rtol=1e-13, atol=1e-13)


def test_grouped_mm_skips_empty_segments():
    asked = []

    def w_of(g):
        asked.append(g)
        return np.ones((2, 3))
    oracle.grouped_mm(np.ones((4, 3)), w_of, [0, 2, 2, 4])
    assert asked == [1, 3]


# ------------------------------------------------------------------ forward vs independent formulations
def torch_mlp(x, wg, wu, wd):
    x, wg, wu, wd = (torch.as_tensor(np.asarray(v, dtype=np.float64)) for v in (x, wg, wu, wd))
    return (torch.nn.functional.silu(x @ wg.T) * (x @ wu.T)) @ wd.T


@pytest.mark.parametrize("seed", range(3))
def test_top1_weight1_is_dense_mlp(seed):
    x, _, _, wg, wu, wd = rand_problem(seed, T=5, E=3, k=1)
    for e in range(3):
        ids = np.full((5, 1), e, dtype=np.int32)
        w = np.ones((5, 1), dtype=np.float32)
        got = oracle.experts_forward(x, ids, w, wg, wu, wd)
        want = torch_mlp(x, wg[e], wu[e], wd[e]).numpy()
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(3))
def test_all_experts_selected_is_dense_mixture(seed):
    # k = E: every expert on every token; compare with a dense einsum over experts
    T, H, I, E = 4, 16, 24, 3
    x, ids, w, wg, wu, wd = rand_problem(seed, T=T, H=H, I=I, E=E, k=E)
    got = oracle.experts_forward(x, ids, w, wg, wu, wd)
    X = torch.as_tensor(x, dtype=torch.float64)
    G = torch.einsum("th,eih->tei", X, torch.as_tensor(wg, dtype=torch.float64))
    U = torch.einsum("th,eih->tei", X, torch.as_tensor(wu, dtype=torch.float64))
    Y = torch.einsum("tei,ehi->teh", torch.nn.functional.silu(G) * U, torch.as_tensor(wd, dtype=torch.float64))
    Wd = torch.zeros(T, E, dtype=torch.float64)
    for t in range(T):
        for j in range(E):
            Wd[t, int(ids[t, j])] = float(w[t, j])
    want = torch.einsum("te,teh->th", Wd, Y).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("act", ["silu", "swiglu_oai", "situ"])
@pytest.mark.parametrize("seed", range(3))
def test_grouped_form_equals_literal_loop(act, seed):
    x, ids, w, wg, wu, wd = rand_problem(seed, T=9, E=5, k=3, masked=0.2, dup=(seed == 2))
    kw = dict(act=act, alpha=1.702 if act != "situ" else 1.5, beta=1.0 if act != "situ" else 2.0,
              limit=2.0 if act == "swiglu_oai" else math.inf)
    a = oracle.experts_forward(x, ids, w, wg, wu, wd, **kw)
    b = oracle.experts_forward_literal(x, ids, w, wg, wu, wd, **kw)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_token_permutation_invariance_bitwise():
    x, ids, w, wg, wu, wd = rand_problem(11, T=12, E=5, k=2)
    pi = np.random.default_rng(0).permutation(12)
    a = oracle.experts_forward(x, ids, w, wg, wu, wd)
    b = oracle.experts_forward(x[pi], ids[pi], w[pi], wg, wu, wd)
    assert np.array_equal(a[pi], b)


def test_route_weight_power_of_two_scales_bitwise():
    x, ids, w, wg, wu, wd = rand_problem(12, T=7, E=4, k=2)
    a = oracle.experts_forward(x, ids, w, wg, wu, wd)
    b = oracle.experts_forward(x, ids, w * 2, wg, wu, wd)
    assert np.array_equal(2 * a, b)


def test_masked_and_bad_ids_contribute_nothing():
    x, ids, w, wg, wu, wd = rand_problem(13, T=8, E=4, k=3)
    ids2 = ids.copy()
    ids2[0, 1] = -1
    ids2[3, 0] = 7                                       # out of range: skipped, counted
    w0 = w.copy()
    w0[0, 1] = 0.0
    w0[3, 0] = 0.0
    a = oracle.experts_forward(x, ids2, w, wg, wu, wd)
    b = oracle.experts_forward(x, ids, w0, wg, wu, wd)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-15)
    assert oracle.align(ids2, 4)["n_bad"] == 1


def test_zero_route_weight_and_empty_input():
    x, ids, w, wg, wu, wd = rand_problem(14, T=3, E=2, k=1)
    out = oracle.experts_forward(x, ids, np.zeros_like(w), wg, wu, wd)
    assert np.all(out == 0)
    out = oracle.experts_forward(x, np.full_like(ids, -1), w, wg, wu, wd)
    assert out.shape == (3, 32) and np.all(out == 0)


def test_combine_is_ascending_j():
    # three slots of one token on one expert with weights 1, 2^40, -2^40:
    # ((y + 2^40 y) - 2^40 y) loses y's low bits, the reverse order keeps y
    x, _, _, wg, wu, wd = rand_problem(15, T=1, E=1, k=1)
    ids = np.zeros((1, 3), dtype=np.int32)
    w = np.array([[1.0, 2.0 ** 40, -(2.0 ** 40)]], dtype=np.float32)
    y = oracle.experts_forward(x, ids[:, :1], w[:, :1], wg, wu, wd)[0]
    got = oracle.experts_forward(x, ids, w, wg, wu, wd)[0]
    want = np.array([((0.0 + v) + v * 2.0 ** 40) + v * -(2.0 ** 40) for v in y])
    assert np.array_equal(got, want)
    assert not np.array_equal(got, y)                   # order is observable here


def test_pregrouped_equals_top1_token_major_and_zero_tail():
    rng = np.random.default_rng(5)
    G, H, I = 5, 16, 24
    lengths = np.array([3, 0, 4, 1, 0])
    NvS = int(lengths.sum()) + 3                         # 3 padding rows past the end
    cu = np.cumsum(lengths)
    x = rng.standard_normal((NvS, H))
    rw = rng.random(NvS)
    wg = rng.standard_normal((G, I, H)) / 4
    wu = rng.standard_normal((G, I, H)) / 4
    wd = rng.standard_normal((G, H, I)) / 5
    got = oracle.pregrouped_forward(x, cu, rw, wg, wu, wd)
    seg = np.repeat(np.arange(G), lengths)
    ids = np.full((NvS, 1), -1, dtype=np.int32)
    ids[: seg.size, 0] = seg
    want = oracle.experts_forward_literal(x, ids, rw[:, None], wg, wu, wd)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    assert np.all(got[int(cu[-1]):] == 0)


# ------------------------------------------------------------------ activations
def test_swiglu_oai_reduces_to_silu_gate():
    g = np.linspace(-9, 9, 101)
    u = np.linspace(3, -4, 101)
    got = oracle.swiglu_oai(g, u, alpha=1.0, beta=0.0, limit=math.inf)
    want = (torch.nn.functional.silu(torch.as_tensor(g)) * torch.as_tensor(u)).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-14)


def test_swiglu_oai_closed_forms():
    a, b, L = 1.702, 1.0, 7.0
    # gate at or above the limit is capped there; up beyond +-limit is flat
    for g in (7.0, 8.5, 100.0):
        for u in (-50.0, -7.0, 0.3, 7.0, 9.0):
            uc = max(-L, min(L, u))
            want = L / (1 + math.exp(-a * L)) * (uc + b)
            assert oracle.swiglu_oai(g, u, a, b, L) == pytest.approx(want, rel=1e-14)
    # below the limit the gate is not clamped from below (one-sided)
    g, u = -30.0, 2.0
    assert oracle.swiglu_oai(g, u, a, b, L) == pytest.approx(g / (1 + math.exp(-a * g)) * (u + b), rel=1e-14)
    assert oracle.swiglu_oai(0.0, 5.0, a, b, L) == 0.0
    # beta shifts the linear branch: u = -beta kills the output
    assert oracle.swiglu_oai(3.0, -b, a, b, L) == 0.0


def test_situ_closed_forms():
    # both factors odd in their argument; g = 0 or u = 0 gives 0
    assert oracle.situ(0.0, 1.3, 2.0, 3.0) == 0.0
    assert oracle.situ(1.1, 0.0, 2.0, 3.0) == 0.0
    g, u, al, be = 0.7, -1.9, 2.5, 1.5
    v = oracle.situ(g, u, al, be)
    assert v == pytest.approx(al * math.tanh(g / al) / (1 + math.exp(-g)) * be * math.tanh(u / be), rel=1e-14)
    # large alpha and beta: alpha*tanh(g/alpha) -> g and beta*tanh(u/beta) -> u, so SiTu -> silu(g)*u
    gg = np.linspace(-3, 3, 13)
    uu = np.linspace(2, -2, 13)
    np.testing.assert_allclose(oracle.situ(gg, uu, 1e5, 1e5),
                               torch.nn.functional.silu(torch.as_tensor(gg)).numpy() * uu, rtol=1e-8, atol=1e-9)


# ------------------------------------------------------------------ MXFP4
def load_e2m1_table():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                c, v = line.split()
                vals[int(c)] = float(v)
    return vals


def test_mxfp4_decode_exhaustive_codes_and_scales():
    table = load_e2m1_table()
    assert len(table) == 16
    # every (low code, high code) byte with every scale byte
    codes = np.arange(256, dtype=np.uint8)
    for v in range(256):
        row = np.repeat(codes[None, :], 1, axis=0)               # [1, 256] bytes = 512 elements
        scales = np.full((1, 512 // 32), v, dtype=np.uint8)
        got = oracle.mxfp4_decode(row, scales)[0]
        if v == 255:
            assert np.all(np.isnan(got))
            continue
        sc = 2.0 ** (v - 127)
        want = np.empty(512)
        for byte in range(256):
            want[2 * byte] = table[byte & 0xF] * sc              # low nibble = element 2i
            want[2 * byte + 1] = table[byte >> 4] * sc
        assert np.array_equal(got, want)
        assert np.array_equal(np.signbit(got), np.signbit(want))


def test_mxfp4_scale_blocks_cover_32_elements():
    codes = np.full((1, 32), 0x22, dtype=np.uint8)              # 64 elements of value 1.0
    scales = np.array([[127 + 3, 127 - 2]], dtype=np.uint8)
    got = oracle.mxfp4_decode(codes, scales)[0]
    assert np.all(got[:32] == 8.0) and np.all(got[32:] == 0.25)


def test_mxfp4_forward_equals_forward_on_decoded_weights():
    rng = np.random.default_rng(21)
    T, H, I, E, k = 5, 64, 96, 4, 2
    x = rng.standard_normal((T, H))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k))

    def q(N, K):
        return (rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8),
                (127 - rng.integers(0, 9, size=(E, N, K // 32))).astype(np.uint8))
    wg, wu, wd = q(I, H), q(I, H), q(H, I)
    kw = dict(act="swiglu_oai", alpha=1.702, beta=1.0, limit=7.0)
    a = oracle.experts_forward(x, ids, w, wg, wu, wd, **kw)
    dec = [np.stack([oracle.mxfp4_decode(c[e], s[e]) for e in range(E)]) for c, s in (wg, wu, wd)]
    b = oracle.experts_forward_literal(x, ids, w, *dec, **kw)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-9)
    # decoded values are exactly bf16-representable for scale bytes 119..127
    d = torch.as_tensor(dec[0])
    assert torch.equal(d.to(torch.bfloat16).to(torch.float64), d)


# ------------------------------------------------------------------ planted mistakes
def _pins_fail(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_planted_mistakes_are_caught(monkeypatch):
    """Each plausible oracle mistake makes at least one pin fail."""
    cases = []
    orig_silu, orig_decode, orig_align = oracle.moe_oracle.silu, oracle.moe_oracle.mxfp4_decode, oracle.moe_oracle.align

    # 1. dropped sigmoid in silu
    cases.append(("silu", lambda g: np.asarray(g, dtype=np.float64),
                  lambda: test_top1_weight1_is_dense_mlp(0)))
    # 2. exponent bias 0 instead of 1 in e2m1 (doubles every normal value)
    def bad_decode(codes, scales):
        v = orig_decode(codes, scales)
        return np.where(np.abs(v) >= np.repeat(np.ldexp(1.0, np.asarray(scales, np.int64) - 127), 32, axis=-1), 2 * v, v)
    cases.append(("mxfp4_decode", bad_decode, test_mxfp4_decode_exhaustive_codes_and_scales))
    # 3. nibble order swapped
    def swapped_decode(codes, scales):
        c = np.asarray(codes, dtype=np.uint8)
        return orig_decode(((c & 0xF) << 4) | (c >> 4), scales)
    cases.append(("mxfp4_decode", swapped_decode, test_mxfp4_decode_exhaustive_codes_and_scales))
    # 4. unstable order inside segments (descending slot index)
    def bad_align(ids, E):
        r = orig_align(ids, E)
        perm = r["perm"].copy()
        s = 0
        for e in range(E):
            perm[s:r["cu_seqlens"][e]] = perm[s:r["cu_seqlens"][e]][::-1]
            s = r["cu_seqlens"][e]
        inv = np.full_like(r["inv_perm"], -1)
        inv[perm] = np.arange(perm.size)
        return dict(r, perm=perm, inv_perm=inv)
    cases.append(("align", bad_align, lambda: test_align_matches_brute_force(0)))

    for attr, bad, pin in cases:
        with monkeypatch.context() as m:
            m.setattr(oracle.moe_oracle, attr, bad)
            m.setattr(oracle, attr, bad)
            assert _pins_fail(pin), f"planted mistake in {attr} went unnoticed"


def test_planted_index_and_operand_mistakes_are_caught(monkeypatch):
    # 5. transposed weight operand (square experts so shapes still fit)
    orig = oracle.moe_oracle.expert_matrix
    with monkeypatch.context() as m:
        m.setattr(oracle.moe_oracle, "expert_matrix", lambda w, e: orig(w, e).T.copy())
        x, _, _, wg, wu, wd = rand_problem(0, T=4, H=24, I=24, E=2, k=1)
        ids = np.zeros((4, 1), dtype=np.int32)
        got = oracle.experts_forward(x, ids, np.ones((4, 1), np.float32), wg, wu, wd)
        assert not np.allclose(got, torch_mlp(x, wg[0], wu[0], wd[0]).numpy(), rtol=1e-6)
    # 6. dropped up projection
    orig_act = oracle.moe_oracle.activation
    with monkeypatch.context() as m:
        m.setattr(oracle.moe_oracle, "activation", lambda n, g, u, *a: oracle.moe_oracle.silu(g))
        assert _pins_fail(lambda: test_top1_weight1_is_dense_mlp(1))
    # 7. wrong sign in the up clamp (clip to [0, limit])
    orig_sw = oracle.moe_oracle.swiglu_oai
    with monkeypatch.context() as m:
        m.setattr(oracle.moe_oracle, "swiglu_oai",
                  lambda g, u, a, b, L: orig_sw(g, np.clip(u, 0, L), a, b, L))
        assert _pins_fail(lambda: test_swiglu_oai_closed_forms_via_module())
    # 8. combine in descending j
    with monkeypatch.context() as m:
        def rev_forward(x, ids, w, *rest, **kw):
            return orig_forward(x, ids[:, ::-1].copy(), w[:, ::-1].copy(), *rest, **kw)
        orig_forward = oracle.moe_oracle.experts_forward
        m.setattr(oracle, "experts_forward", rev_forward)
        assert _pins_fail(test_combine_is_ascending_j)


def test_swiglu_oai_closed_forms_via_module():
    f = oracle.moe_oracle.swiglu_oai
    a, b, L = 1.702, 1.0, 7.0
    for g in (7.0, 100.0):
        for u in (-50.0, -3.0, 9.0):
            uc = max(-L, min(L, u))
            assert f(g, u, a, b, L) == pytest.approx(L / (1 + math.exp(-a * L)) * (uc + b), rel=1e-14)


# ------------------------------------------------------------------ route weight on the input
@pytest.mark.parametrize("seed", range(3))
def test_weight_on_input_top1_is_dense_mlp_of_scaled_input(seed):
    """Top-1 with the route weight on the input: a dense SwiGLU MLP (torch silu)
    applied to w * x (moonep_experts page: input-weighted routing scales the
    activations before dispatch)."""
    x, _, _, wg, wu, wd = rand_problem(seed, T=5, E=3, k=1)
    rng = np.random.default_rng(seed + 10)
    w = rng.uniform(0.1, 2.0, (5, 1)).astype(np.float32)
    for e in range(3):
        ids = np.full((5, 1), e, dtype=np.int32)
        got = oracle.experts_forward(x, ids, w, wg, wu, wd, weight_on_input=True)
        want = torch_mlp(x * w.astype(np.float64), wg[e], wu[e], wd[e]).numpy()
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
        # differs from the output-side weighting (silu is not homogeneous)
        other = oracle.experts_forward(x, ids, w, wg, wu, wd)
        assert not np.allclose(got, other, rtol=1e-3)


def test_weight_on_input_grouped_equals_literal():
    x, ids, w, wg, wu, wd = rand_problem(4, T=7, E=4, k=2)
    for act, kw in (("silu", {}), ("situ", dict(alpha=1.5, beta=0.8))):
        a = oracle.experts_forward(x, ids, w, wg, wu, wd, act=act, weight_on_input=True, **kw)
        b = oracle.experts_forward_literal(x, ids, w, wg, wu, wd, act=act, weight_on_input=True, **kw)
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_situ_forward_top1_is_dense_situ_mlp():
    """SiTu through the whole forward equals a dense MLP written with torch's
    tanh and sigmoid from the page's formula: alpha*tanh(g/alpha)*sigmoid(g)
    times beta*tanh(u/beta)."""
    x, _, _, wg, wu, wd = rand_problem(2, T=4, E=2, k=1)
    al, be = 1.7, 0.6
    ids = np.ones((4, 1), dtype=np.int32)
    got = oracle.experts_forward(x, ids, np.ones((4, 1), np.float32), wg, wu, wd, act="situ", alpha=al, beta=be)
    X, G, U, D = (torch.as_tensor(np.asarray(v, dtype=np.float64)) for v in (x, wg[1], wu[1], wd[1]))
    g, u = X @ G.T, X @ U.T
    want = ((al * torch.tanh(g / al) * torch.sigmoid(g)) * (be * torch.tanh(u / be))) @ D.T
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ MXFP8 activations
def _e4m3_table():
    """All finite e4m3 (fn) values from their bit patterns: sign, 4 exponent
    bits (bias 7), 3 mantissa bits; exponent 15 with mantissa 7 is NaN."""
    vals = {}
    for code in range(256):
        s, e, m = code >> 7, (code >> 3) & 15, code & 7
        if e == 15 and m == 7:
            continue
        mag = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
        vals[code] = -mag if s else mag
    return vals


def test_e4m3_round_exhaustive_grid_midpoints_and_saturation():
    table = _e4m3_table()
    grid = np.array(sorted({v for v in table.values() if v >= 0}))
    assert grid[-1] == 448.0 and len(grid) == 127
    assert np.array_equal(oracle.e4m3_round(grid), grid)
    assert np.array_equal(oracle.e4m3_round(-grid), -grid)
    # a midpoint goes to the neighbour whose mantissa bit 0 is clear
    even = {v: (c & 1) == 0 for c, v in table.items() if v >= 0}
    lo, hi = grid[:-1], grid[1:]
    mid = (lo + hi) / 2
    want = np.where([even[a] for a in lo], lo, hi)
    assert np.array_equal(oracle.e4m3_round(mid), want)
    # just off the midpoint goes to the nearer neighbour
    assert np.array_equal(oracle.e4m3_round(mid - (hi - lo) * 1e-3), lo)
    assert np.array_equal(oracle.e4m3_round(mid + (hi - lo) * 1e-3), hi)
    big = np.array([448.5, 463.9, 464.0, 480.0, 1e6])
    assert np.array_equal(oracle.e4m3_round(big), np.full(5, 448.0))
    assert np.array_equal(oracle.e4m3_round(-big), np.full(5, -448.0))


def test_e4m3_round_matches_torch_float8_in_range():
    # torch's float8_e4m3fn conversion (round to nearest even) on float32
    # inputs inside the finite range
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.uniform(-4, 2.5, 20000),
                        rng.uniform(-448, 448, 5000)]).astype(np.float32)
    v = v[np.abs(v) <= 448]          # torch gives NaN past the range; the oracle saturates
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(oracle.e4m3_round(v.astype(np.float64)), ref)


def test_mxfp8_quantize_closed_forms():
    # amax 1 -> X = 2^-8 (code 119): 0.1 * 256 = 25.6 lies in [16, 32), spacing 2 -> 26
    v, e, c = oracle.mxfp8_quantize(np.array([[1.0, 0.1, 0.01] + [0.0] * 29]))
    assert c.tolist() == [[119]]
    assert v[0, :3].tolist() == [1.0, 26 / 256, 2.5 / 256]
    assert e[0, :3].tolist() == [256.0, 26.0, 2.5]
    # amax 1.9: 1.9 * 256 = 486.4 saturates at 448 -> 1.75
    v, e, c = oracle.mxfp8_quantize(np.array([[-1.9] + [0.25] * 31]))
    assert c.tolist() == [[119]] and v[0, 0] == -1.75 and e[0, 0] == -448.0 and v[0, 1] == 0.25
    # an all-zero block: code 0, zeros; scale codes clamp at both ends
    v, e, c = oracle.mxfp8_quantize(np.zeros((1, 64)))
    assert c.tolist() == [[0, 0]] and not v.any()
    _, _, c = oracle.mxfp8_quantize(np.array([[2.0 ** -130] + [0.0] * 31, [2.0 ** 200] + [0.0] * 31]))
    assert c.ravel().tolist() == [0, 254]
    with pytest.raises(ValueError):
        oracle.mxfp8_quantize(np.zeros((2, 48)))


def test_mxfp8_values_on_the_grid_are_fixed_points():
    # blocks built as e4m3 values times 2^(c-127), with one element in
    # [256, 448] so that the block's own scale is 2^(c-127): unchanged
    rng = np.random.default_rng(4)
    grid = np.array(sorted(set(_e4m3_table().values())))
    top = grid[(np.abs(grid) >= 256)]
    rows = []
    codes = rng.integers(1, 240, size=40)
    for c in codes:
        el = rng.choice(grid, size=32)
        el = np.where(np.abs(el) > 448, 448.0, el)
        el[rng.integers(32)] = rng.choice(top)
        rows.append(el * 2.0 ** (int(c) - 127))
    a = np.array(rows)
    v, e, cq = oracle.mxfp8_quantize(a)
    assert np.array_equal(v, a)
    assert cq.ravel().tolist() == codes.tolist()


def test_mxfp8_error_bound_on_random_rows():
    rng = np.random.default_rng(5)
    a = rng.standard_normal((64, 256)) * 10.0 ** rng.uniform(-3, 3, (64, 1))
    v, e, c = oracle.mxfp8_quantize(a)
    X = np.repeat(np.ldexp(1.0, c.astype(np.int32) - 127), 32, axis=-1)
    r = np.abs(a) / X
    err = np.abs(v - a) / X
    _, ex = np.frexp(r)
    half_ulp = np.ldexp(1.0, np.maximum(ex - 1, -6) - 4)    # half the spacing 2^(b-3)
    sat = r > 448
    assert np.all(err[~sat] <= half_ulp[~sat])
    # saturation happens only in blocks whose amax / X reaches 464 (mantissa >= 1.8125)
    assert np.all(r[sat] >= 448)
    assert np.all(np.abs(e) <= 448)


def test_mxfp8_forward_grouped_equals_literal_and_differs_from_exact():
    x, ids, w, wg, wu, wd = rand_problem(21, T=7, H=64, I=96, E=4, k=2, masked=0.2)
    for woi in (False, True):
        a = oracle.experts_forward(x, ids, w, wg, wu, wd, weight_on_input=woi, act_fmt="mxfp8")
        b = oracle.experts_forward_literal(x, ids, w, wg, wu, wd, weight_on_input=woi, act_fmt="mxfp8")
        assert np.max(np.abs(a - b)) <= 1e-12 * np.max(np.abs(b))
        exact = oracle.experts_forward(x, ids, w, wg, wu, wd, weight_on_input=woi)
        d = np.max(np.abs(a - exact)) / np.max(np.abs(exact))
        assert 1e-4 < d < 0.1        # e4m3 keeps 4 significant bits
    # on-grid inputs are not changed by the first quantization: with the
    # activation left exact, gate and up see x itself
    with pytest.raises(ValueError):
        oracle.experts_forward(x, ids, w, wg, wu, wd, act_fmt="fp4")


def test_bf16_round_matches_torch_and_closed_forms():
    # torch's float32 -> bfloat16 conversion (round to nearest even) on float32 inputs
    rng = np.random.default_rng(8)
    v = (rng.standard_normal(50000) * 10.0 ** rng.uniform(-20, 20, 50000)).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.bf16_round(v.astype(np.float64)), ref)
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7: ties to even (1); just above goes up
    assert oracle.bf16_round(np.array([1 + 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, 3 * 2.0 ** -9 + 1])).tolist() == \
        [1.0, 1 + 2.0 ** -7, 1 + 2.0 ** -7]
    assert oracle.bf16_round(np.array([0.0, -2.0 ** 100])).tolist() == [0.0, -2.0 ** 100]


def test_mxfp8_mode_rounds_token_rows_to_bf16_but_not_activation_rows():
    # bf16 values are unchanged by the bf16 rounding, so on bf16 token rows the
    # mode's first quantization is exactly mxfp8_quantize
    rng = np.random.default_rng(9)
    rows = torch.from_numpy(rng.standard_normal((4, 64)).astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(oracle.moe_oracle._act_in(rows, "mxfp8", bf16_first=True), oracle.mxfp8_quantize(rows)[0])
    # an off-grid value that bf16 rounding moves onto an e4m3 midpoint: in a
    # block of amax 1.5 (scale 2^-8) the e4m3 neighbours of 1 + 2^-4 are 1 and
    # 1 + 2^-3; 1 + 2^-4 + 2^-10 rounds to 1 + 2^-4 in bf16 (8 bits), then to 1
    # (even) in e4m3, while unrounded it goes up to 1 + 2^-3. Token rows (a
    # bf16 tensor, or the weighted rows rounded to bf16) take the first path;
    # activation rows, quantized from their exact value inside the step, the
    # second.
    blk = np.zeros((1, 32))
    blk[0, 0] = 1.5
    blk[0, 1] = 1 + 2.0 ** -4 + 2.0 ** -10
    assert oracle.moe_oracle._act_in(blk, "mxfp8", bf16_first=True)[0, 1] == 1.0
    assert oracle.moe_oracle._act_in(blk, "mxfp8", bf16_first=False)[0, 1] == 1 + 2.0 ** -3
    assert oracle.mxfp8_quantize(blk)[0][0, 1] == 1 + 2.0 ** -3


# ------------------------------------------------------------------ per-expert parameters
def test_per_expert_params_equal_scalars_when_constant():
    x, ids, w, wg, wu, wd = rand_problem(31, T=9, H=32, I=64, E=4, k=2, masked=0.1)
    kw = dict(act="swiglu_oai", alpha=1.702, beta=1.0, limit=7.0)
    a = oracle.experts_forward(x, ids, w, wg, wu, wd, **kw)
    b = oracle.experts_forward(x, ids, w, wg, wu, wd, act="swiglu_oai", alpha=np.full(4, 1.702),
                               beta=np.full(4, 1.0), limit=np.full(4, 7.0), fc1_alpha=np.ones(4), fc2_alpha=np.ones(4))
    assert np.array_equal(a, b)


def test_fc1_fc2_alphas_equal_prescaled_weights_in_a_dense_torch_mlp():
    # top-1, weight 1: each token's output is its expert's MLP, so scaling the
    # gate / up products by fc1[e] and the down product by fc2[e] must equal a
    # dense torch MLP whose weights were multiplied by those scales
    x, ids, w, wg, wu, wd = rand_problem(32, T=12, H=32, I=64, E=3, k=1)
    w[:] = 1.0
    fc1 = np.array([0.7, 1.9, 0.25])
    fc2 = np.array([3.0, 0.5, 1.3])
    got = oracle.experts_forward(x, ids, w, wg, wu, wd, fc1_alpha=fc1, fc2_alpha=fc2)
    X = torch.from_numpy(x.astype(np.float64))
    for t in range(12):
        e = int(ids[t, 0])
        g = X[t] @ torch.from_numpy(wg[e].astype(np.float64) * fc1[e]).T
        u = X[t] @ torch.from_numpy(wu[e].astype(np.float64) * fc1[e]).T
        ref = (torch.nn.functional.silu(g) * u) @ torch.from_numpy(wd[e].astype(np.float64) * fc2[e]).T
        assert np.allclose(got[t], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_per_expert_activation_params_are_the_union_of_scalar_runs():
    # distinct alpha / beta / limit per expert: every token of a top-1
    # problem gets exactly what the scalar oracle gives with its expert's values
    x, ids, w, wg, wu, wd = rand_problem(33, T=16, H=32, I=64, E=4, k=1)
    x = x * 3.0                      # reach the clamp limits
    al = np.array([1.702, 0.5, 2.5, 1.0])
    be = np.array([1.0, 0.0, -0.5, 2.0])
    li = np.array([7.0, 0.3, np.inf, 1.5])
    got = oracle.experts_forward(x, ids, w, wg, wu, wd, act="swiglu_oai", alpha=al, beta=be, limit=li)
    lit = oracle.experts_forward_literal(x, ids, w, wg, wu, wd, act="swiglu_oai", alpha=al, beta=be, limit=li)
    assert np.max(np.abs(got - lit)) <= 1e-12 * np.max(np.abs(lit))
    for e in range(4):
        rows = np.where(ids[:, 0] == e)[0]
        if len(rows) == 0:
            continue
        ref = oracle.experts_forward(x[rows], ids[rows], w[rows], wg, wu, wd, act="swiglu_oai", alpha=al[e],
                                     beta=be[e], limit=li[e])
        assert np.array_equal(got[rows], ref)
    # the experts' values really differ in effect
    same = oracle.experts_forward(x, ids, w, wg, wu, wd, act="swiglu_oai", alpha=1.702, beta=1.0, limit=7.0)
    assert np.max(np.abs(got - same)) > 1e-3 * np.max(np.abs(same))
