"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test ties one oracle function to a library routine, a closed form, an
exactly rounded brute-force sum or an invariant the mathematics fixes, so that
a dropped term, a wrong sign, a wrong index or a transposed operand fails.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import expit, softmax

import oracle
import synth

# ----------------------------------------------------------------- helpers


def f16(a):
    return np.asarray(a, dtype=np.float32).astype(np.float16)


def bits16(a_f16):
    return np.ascontiguousarray(a_f16).view(np.uint16)


def unpack_codes(up_q, d):
    """Codes [f][d] from the INT2 rows: little-endian 32-bit words of 16 codes,
    input 16i + 2m + h in bits 16h + 2m of word i."""
    w = np.ascontiguousarray(up_q).view("<u4").astype(np.int64)     # [f][d/16]
    k = np.arange(d)
    shift = 16 * (k % 2) + 2 * ((k % 16) // 2)
    return (w[:, k // 16] >> shift) & 3


def exact_int2_expert(rng, d, f, s_pow=-7):
    """Up weights that INT2 represents exactly: per (channel, group) pick
    codes with 0 and 3 both present, s = 2^s_pow, z in {0.5,1,1.5,2}, and
    w = s*(q - z).  Returns (w_t f32 [f][d], codes [f][d], s, z [f][d/64])."""
    G = d // 64
    q = rng.integers(0, 4, size=(f, d))
    q[:, ::64] = 0
    q[:, 1::64] = 3
    z = rng.choice(np.array([0.5, 1.0, 1.5, 2.0]), size=(f, G))
    s = 2.0 ** s_pow
    w = s * (q - np.repeat(z, 64, axis=1))
    w32 = w.astype(np.float32)
    assert np.all(w32.astype(np.float64) == w)
    return w32, q, s, z


# ----------------------------------------------------------------- scalars

def test_half_to_double_all_patterns():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = b.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(v)) for v in b])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_to_double_all_patterns():
    b = np.arange(65536, dtype=np.int32).astype(np.int16)
    ref = torch.from_numpy(b.copy()).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_to_double(int(v) & 0xFFFF) for v in b])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_double_to_half_rne_matches_numpy():
    rng = np.random.default_rng(5)
    vals = np.concatenate([
        rng.standard_normal(4000) * 10.0 ** rng.uniform(-9, 5, 4000),
        # exact ties between neighbours: midpoints of consecutive halves
        (np.arange(1, 2000, dtype=np.uint16).view(np.float16).astype(np.float64)
         + np.arange(2, 2001, dtype=np.uint16).view(np.float16).astype(np.float64)) / 2,
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
         2.0 ** -14, 2.0 ** -14 - 2.0 ** -25],
    ])
    with np.errstate(over="ignore"):
        ref = bits16(vals.astype(np.float16))
    got = np.array([oracle.double_to_half_rne(v) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_double_to_bf16_rne_matches_torch_on_float_values():
    rng = np.random.default_rng(6)
    vals = (rng.standard_normal(5000) * 10.0 ** rng.uniform(-30, 30, 5000)).astype(np.float32)
    # halfway cases: exactly between two bf16 neighbours
    base = (rng.integers(0x3000, 0x5000, 500).astype(np.uint32) << 16)
    ties = (base | 0x8000).view(np.float32)
    vals = np.concatenate([vals, ties, np.float32([0.0, 1.0, -2.5, 3e38])])
    ref = torch.from_numpy(vals.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.double_to_bf16_rne(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_double_to_bf16_rne_single_rounding():
    # 1 + 2^-8 + 2^-30 lies just above the bf16 midpoint 1 + 2^-8: the correct
    # rounding goes up (0x3F81); rounding through float32 first would land on
    # the midpoint and tie to even (0x3F80).
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert oracle.double_to_bf16_rne(v) == 0x3F81
    assert oracle.double_to_bf16_rne(1.0 + 2.0 ** -8) == 0x3F80


# ----------------------------------------------------------------- INT2 format

def test_pack_exact_weights_round_trip():
    rng = np.random.default_rng(7)
    d, f = 256, 9
    w, q, s, z = exact_int2_expert(rng, d, f)
    up_q, up_sz = oracle.pack_up_int2(w)
    # scales and zeros are exactly the ones used to build the weights
    assert np.all(up_sz[..., 0] == bits16(f16(np.full((f, d // 64), s))))
    assert np.all(up_sz[..., 1] == bits16(f16(z)))
    assert np.array_equal(unpack_codes(up_q, d), q)
    # dequantisation gives the original weights back exactly
    assert np.array_equal(oracle.dequant_up(up_q, up_sz, d), w.astype(np.float64))


def test_pack_code_layout_single_code():
    d = 64
    for k in (0, 1, 2, 3, 5, 37, 63):
        w = np.zeros((1, d), dtype=np.float32)
        w[0, k] = 3.0          # group min 0, max 3 -> s = 1, z = 0
        up_q, up_sz = oracle.pack_up_int2(w)
        # input 16i + 2m + h -> bits 16h + 2m of little-endian word i
        i, m, h = k // 16, (k % 16) // 2, k % 2
        bit = 32 * i + 16 * h + 2 * m
        expect = np.zeros(d // 4, dtype=np.uint8)
        expect[bit // 8] = 3 << (bit % 8)
        assert np.array_equal(up_q[0], expect), k
        # -mn = -0.0 for a group whose minimum is +0, so z is the fp16 -0
        assert up_sz[0, 0, 0] == 0x3C00 and up_sz[0, 0, 1] in (0, 0x8000)


def test_pack_error_bound_and_extremes():
    w = synth.normal_f32(12345, (64, 512), 0.02)
    up_q, up_sz = oracle.pack_up_int2(w)
    deq = oracle.dequant_up(up_q, up_sz, 512)
    s = np.repeat(np.asarray([[oracle.half_to_double(b) for b in row] for row in up_sz[..., 0]]), 64, 1)
    err = np.abs(deq - w.astype(np.float64))
    # half a step plus the fp16 rounding of s and z (each < 2^-11 relative)
    assert np.all(err <= 0.5 * s + 4 * s * 2.0 ** -11 + 1e-12)
    codes = unpack_codes(up_q, 512)
    g = w.reshape(64, 8, 64)
    cg = codes.reshape(64, 8, 64)
    amin = g.argmin(-1)
    amax = g.argmax(-1)
    assert np.all(np.take_along_axis(cg, amin[..., None], -1) == 0)
    assert np.all(np.take_along_axis(cg, amax[..., None], -1) == 3)


def test_pack_constant_group_uses_unit_scale():
    w = np.full((2, 64), 0.25, dtype=np.float32)
    up_q, up_sz = oracle.pack_up_int2(w)
    assert np.all(up_sz[:, 0, 0] == 0x3C00)   # s = 1 when (mx-mn)/3 rounds to 0
    deq = oracle.dequant_up(up_q, up_sz, 64)
    assert np.all(np.abs(deq - 0.25) <= 0.5)


def test_materialize_up_bf16_exact_values():
    rng = np.random.default_rng(8)
    d, f = 128, 5
    G = d // 64
    q = rng.integers(0, 4, size=(f, d))
    q[:, ::64] = 0
    q[:, 1::64] = 3
    z = np.ones((f, G))
    w = (2.0 ** -7) * (q - 1.0)
    up_q, up_sz = oracle.pack_up_int2(w.astype(np.float32))
    got = oracle.materialize_up_bf16(up_q, up_sz, d)
    ref = torch.from_numpy(w.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


# ----------------------------------------------------------------- one expert

def _tiny_expert(seed, d=128, f=96, wdt="f16", exact=False):
    rng = np.random.default_rng(seed)
    if exact:
        w_up, _, _, _ = exact_int2_expert(rng, d, f)
    else:
        w_up = (rng.standard_normal((f, d)) * 0.02).astype(np.float32)
    up_q, up_sz = oracle.pack_up_int2(w_up)
    g = (rng.standard_normal((f, d)) * 0.02).astype(np.float32)
    dn = (rng.standard_normal((f, d)) * 0.02).astype(np.float32)
    return w_up, up_q, up_sz, synth.to_bits(g, wdt), synth.to_bits(dn, wdt)


def _bits_to_f64(bits, dt):
    if dt == "f16":
        return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_expert_bruteforce_fsum():
    """v, g and y against exactly rounded sums (math.fsum) and math.exp."""
    d, f, T = 64, 40, 2
    w_up, up_q, up_sz, gb, db = _tiny_expert(1, d, f, exact=True)
    x = synth.to_f16_bits(synth.normal_f32(2, (T, d), 1 / 16))
    v, m, y = oracle.expert_forward(x, "f16", up_q, up_sz, gb, db, "f16", thr=0.01)
    X = _bits_to_f64(x, "f16")
    Gm = _bits_to_f64(gb, "f16")
    Dm = _bits_to_f64(db, "f16")
    W = w_up.astype(np.float64)
    assert 0 < m.sum() < T * f
    for t in range(T):
        yref = [[] for _ in range(d)]
        for j in range(f):
            vj = math.fsum(X[t, k] * W[j, k] for k in range(d))
            assert v[t, j] == pytest.approx(vj, rel=1e-13, abs=1e-16)
            assert m[t, j] == (abs(vj) > float(np.float32(0.01)))
            if m[t, j]:
                gj = math.fsum(X[t, k] * Gm[j, k] for k in range(d))
                hj = gj / (1.0 + math.exp(-gj)) * vj
                for c in range(d):
                    yref[c].append(hj * Dm[j, c])
        for c in range(d):
            assert y[t, c] == pytest.approx(math.fsum(yref[c]), rel=1e-11, abs=1e-15)


@pytest.mark.parametrize("wdt", ["f16", "bf16"])
def test_expert_dense_threshold_is_textbook_swiglu(wdt):
    """t < 0 keeps every channel: (SiLU(x W_gate) * (x W_up)) W_down with the
    original (exactly representable) up weights, in numpy float64."""
    d, f, T = 256, 192, 3
    w_up, up_q, up_sz, gb, db = _tiny_expert(3, d, f, wdt=wdt, exact=True)
    x = synth.to_bits(synth.normal_f32(4, (T, d), 1 / 16), wdt)
    v, m, y = oracle.expert_forward(x, wdt, up_q, up_sz, gb, db, wdt, thr=-1.0)
    X = _bits_to_f64(x, wdt)
    Wg = _bits_to_f64(gb, wdt).T            # d x f
    Wd = _bits_to_f64(db, wdt)              # f x d
    Wu = w_up.astype(np.float64).T          # d x f
    ref = (X @ Wg * expit(X @ Wg) * (X @ Wu)) @ Wd
    assert np.all(m == 1)
    np.testing.assert_allclose(v, X @ Wu, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-14)


def test_expert_infinite_threshold_gives_zero():
    _, up_q, up_sz, gb, db = _tiny_expert(5)
    x = synth.to_f16_bits(synth.normal_f32(6, (2, 128), 1 / 16))
    v, m, y = oracle.expert_forward(x, "f16", up_q, up_sz, gb, db, "f16", thr=np.inf)
    assert np.all(m == 0) and np.all(y == 0.0)
    assert np.any(v != 0.0)


def test_expert_single_active_channel_closed_form():
    d, f = 128, 96
    w_up, up_q, up_sz, gb, db = _tiny_expert(7, d, f, exact=True)
    x = synth.to_f16_bits(synth.normal_f32(8, (1, d), 1 / 16))
    X = _bits_to_f64(x, "f16")[0]
    vref = w_up.astype(np.float64) @ X
    order = np.argsort(-np.abs(vref))
    j = order[0]
    thr = np.float32((abs(vref[order[0]]) + abs(vref[order[1]])) / 2)
    v, m, y = oracle.expert_forward(x, "f16", up_q, up_sz, gb, db, "f16", thr=thr)
    assert m.sum() == 1 and m[0, j] == 1
    g = _bits_to_f64(gb, "f16")[j] @ X
    ref = g * expit(g) * vref[j] * _bits_to_f64(db, "f16")[j]
    np.testing.assert_allclose(y[0], ref, rtol=1e-12, atol=1e-16)


def test_expert_mask_additivity_and_monotonicity():
    d, f = 128, 96
    _, up_q, up_sz, gb, db = _tiny_expert(9, d, f)
    x = synth.to_f16_bits(synth.normal_f32(10, (2, d), 1 / 16))
    v, m_lo, y_lo = oracle.expert_forward(x, "f16", up_q, up_sz, gb, db, "f16", thr=0.005)
    _, m_hi, _ = oracle.expert_forward(x, "f16", up_q, up_sz, gb, db, "f16", thr=0.02)
    assert np.all(m_hi <= m_lo) and m_hi.sum() < m_lo.sum()
    rng = np.random.default_rng(11)
    split = (rng.random(m_lo.shape) < 0.5).astype(np.uint8)
    m1 = m_lo & split
    m2 = m_lo & (1 - split)
    _, _, y1 = oracle.expert_forward(x, "f16", up_q, up_sz, gb, db, "f16", 0.0, mask_in=m1)
    _, _, y2 = oracle.expert_forward(x, "f16", up_q, up_sz, gb, db, "f16", 0.0, mask_in=m2)
    np.testing.assert_allclose(y1 + y2, y_lo, rtol=1e-12, atol=1e-16)


def test_expert_channel_permutation_invariance():
    d, f = 128, 96
    _, up_q, up_sz, gb, db = _tiny_expert(12, d, f)
    x = synth.to_f16_bits(synth.normal_f32(13, (3, d), 1 / 16))
    perm = np.random.default_rng(14).permutation(f)
    v, m, y = oracle.expert_forward(x, "f16", up_q, up_sz, gb, db, "f16", thr=0.01)
    vp, mp, yp = oracle.expert_forward(x, "f16", up_q[perm], up_sz[perm], gb[perm], db[perm],
                                       "f16", thr=0.01)
    np.testing.assert_array_equal(vp, v[:, perm])
    np.testing.assert_array_equal(mp, m[:, perm])
    np.testing.assert_allclose(yp, y, rtol=1e-12, atol=1e-16)


def test_expert_tokens_independent_scale_and_accumulate():
    d, f = 128, 96
    _, up_q, up_sz, gb, db = _tiny_expert(15, d, f)
    x = synth.to_f16_bits(synth.normal_f32(16, (4, d), 1 / 16))
    _, _, y = oracle.expert_forward(x, "f16", up_q, up_sz, gb, db, "f16", thr=0.01)
    for t in range(4):
        _, _, yt = oracle.expert_forward(x[t:t + 1], "f16", up_q, up_sz, gb, db, "f16", thr=0.01)
        np.testing.assert_array_equal(yt[0], y[t])
    sc = np.array([0.5, -2.0, 0.0, 3.0])
    y0 = np.arange(4 * d, dtype=np.float64).reshape(4, d)
    _, _, ys = oracle.expert_forward(x, "f16", up_q, up_sz, gb, db, "f16", thr=0.01,
                                     scale=sc, y_init=y0)
    np.testing.assert_allclose(ys, y0 + sc[:, None] * y, rtol=1e-14, atol=1e-15)


def test_silu_odd_part_through_single_channel():
    """SiLU(g) - SiLU(-g) = g: flipping the sign of the gate row turns the
    single-channel output from SiLU(g) v D_j into SiLU(-g) v D_j."""
    d, f = 64, 64
    w_up, up_q, up_sz, gb, db = _tiny_expert(17, d, f, exact=True)
    x = synth.to_f16_bits(synth.normal_f32(18, (1, d), 1 / 16))
    mask = np.zeros((1, f), dtype=np.uint8)
    mask[0, 5] = 1
    v, _, y_pos = oracle.expert_forward(x, "f16", up_q, up_sz, gb, db, "f16", 0.0, mask_in=mask)
    neg = gb.copy()
    neg[5] ^= 0x8000
    _, _, y_neg = oracle.expert_forward(x, "f16", up_q, up_sz, neg, db, "f16", 0.0, mask_in=mask)
    g = _bits_to_f64(gb, "f16")[5] @ _bits_to_f64(x, "f16")[0]
    np.testing.assert_allclose((y_pos - y_neg)[0], g * v[0, 5] * _bits_to_f64(db, "f16")[5],
                               rtol=1e-11, atol=1e-16)
    zero_gate = gb.copy()
    zero_gate[5] = 0
    _, _, y_zero = oracle.expert_forward(x, "f16", up_q, up_sz, zero_gate, db, "f16", 0.0,
                                         mask_in=mask)
    assert np.all(y_zero == 0.0)


# ----------------------------------------------------------------- router

def _router_case(seed, T, d, E, dup=False):
    x = synth.to_f16_bits(synth.normal_f32(seed, (T, d), 1.0))
    R = synth.normal_f32(seed + 1, (E, d), 0.02)
    if dup:
        R[3] = R[1]
        R[E - 1] = R[0]
    return x, synth.to_f16_bits(R)


@pytest.mark.parametrize("renorm", [True, False])
def test_router_against_argsort_and_softmax(renorm):
    T, d, E, k = 33, 128, 16, 4
    x, R = _router_case(20, T, d, E)
    b = synth.zipf_bias(5, 0, E, 1.1)
    out = oracle.route_topk(x, "f16", R, "f16", E, k, renormalize=renorm, bias=b)
    X = _bits_to_f64(x, "f16")
    L = X @ _bits_to_f64(R, "f16").T + b.astype(np.float64)
    np.testing.assert_allclose(out["logits"], L, rtol=1e-12, atol=1e-13)
    ref_idx = np.argsort(-L, axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(out["topk_idx"], ref_idx)
    if renorm:
        ref_w = softmax(np.take_along_axis(L, ref_idx, 1), axis=1)
        np.testing.assert_allclose(out["topk_w"].sum(1), 1.0, rtol=1e-14)
    else:
        ref_w = np.take_along_axis(softmax(L, axis=1), ref_idx, 1)
    np.testing.assert_allclose(out["topk_w"], ref_w, rtol=1e-12)
    flat = ref_idx.ravel()
    np.testing.assert_array_equal(out["expert_count"], np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(out["expert_offset"],
                                  np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    np.testing.assert_array_equal(out["pair_by_expert"], np.argsort(flat, kind="stable"))
    assert out["expert_count"].sum() == T * k       # one row of the activation matrix


def test_router_ties_go_to_lowest_index_and_k_equals_E():
    T, d, E = 8, 64, 8
    x, R = _router_case(30, T, d, E, dup=True)
    out = oracle.route_topk(x, "f16", R, "f16", E, E, renormalize=True)
    L = out["logits"]
    assert np.all(L[:, 3] == L[:, 1]) and np.all(L[:, E - 1] == L[:, 0])
    for t in range(T):
        order = list(out["topk_idx"][t])
        assert sorted(order) == list(range(E))
        assert order.index(1) < order.index(3)
        assert order.index(0) < order.index(E - 1)
        assert np.all(np.diff(L[t, order]) <= 0)
    np.testing.assert_allclose(out["topk_w"], softmax(np.take_along_axis(L, out["topk_idx"], 1), 1))


# ----------------------------------------------------------------- layer

def _tiny_layer(seed, d, f, E, S, wdt="f16"):
    ups, szs, gs, ds = [], [], [], []
    for e in range(E + S):
        _, q, sz, g, dn = _tiny_expert(seed + 7 * e, d, f, wdt=wdt)
        ups.append(q); szs.append(sz); gs.append(g); ds.append(dn)
    return np.stack(ups), np.stack(szs), np.stack(gs), np.stack(ds)


def test_layer_single_expert_reduces_to_expert():
    d, f = 128, 64
    uq, us, g, dn = _tiny_layer(40, d, f, 1, 0)
    x, R = _router_case(41, 3, d, 1)
    y, idx, w, m = oracle.layer_forward(x, "f16", R, "f16", None, 1, 1, 0, True, uq, us, g, dn,
                                        "f16", np.float32([0.01]))
    assert np.all(idx == 0) and np.all(w == 1.0)
    _, me, ye = oracle.expert_forward(x, "f16", uq[0], us[0], g[0], dn[0], "f16", thr=0.01)
    np.testing.assert_array_equal(y, ye)
    np.testing.assert_array_equal(m[:, 0], me)


def test_layer_is_weighted_sum_of_experts_plus_shared():
    d, f, E, k, S, T = 128, 64, 6, 2, 2, 5
    uq, us, g, dn = _tiny_layer(50, d, f, E, S)
    x, R = _router_case(51, T, d, E)
    thr = np.float32([0.01] * (E + S))
    y, idx, w, m = oracle.layer_forward(x, "f16", R, "f16", None, E, k, S, True, uq, us, g, dn,
                                        "f16", thr)
    X = _bits_to_f64(x, "f16")
    L = X @ _bits_to_f64(R, "f16").T
    np.testing.assert_array_equal(idx, np.argsort(-L, 1, kind="stable")[:, :k])
    ref = np.zeros((T, d))
    for t in range(T):
        for s in range(k):
            e = idx[t, s]
            _, _, ye = oracle.expert_forward(x[t:t + 1], "f16", uq[e], us[e], g[e], dn[e], "f16", 0.01)
            ref[t] += w[t, s] * ye[0]
        for i in range(S):
            _, _, ye = oracle.expert_forward(x[t:t + 1], "f16", uq[E + i], us[E + i], g[E + i],
                                             dn[E + i], "f16", 0.01)
            ref[t] += ye[0]
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-16)
    # routed experts switched off (t=+inf): only the shared experts remain
    thr_off = np.float32([np.inf] * E + [0.01] * S)
    y_sh, _, _, m_sh = oracle.layer_forward(x, "f16", R, "f16", None, E, k, S, True, uq, us, g, dn,
                                            "f16", thr_off)
    assert np.all(m_sh[:, :k] == 0)
    sh = np.zeros((T, d))
    for i in range(S):
        _, _, ye = oracle.expert_forward(x, "f16", uq[E + i], us[E + i], g[E + i], dn[E + i], "f16", 0.01)
        sh += ye
    np.testing.assert_allclose(y_sh, sh, rtol=1e-12, atol=1e-16)


def test_layer_dense_path_is_bf16_swiglu():
    d, f, E, k, T = 128, 64, 4, 2, 3
    rng = np.random.default_rng(60)
    ups, szs, gs, ds, ws = [], [], [], [], []
    for e in range(E):
        w, _, _, _ = exact_int2_expert(rng, d, f)
        q, sz = oracle.pack_up_int2(w)
        ups.append(q); szs.append(sz); ws.append(w.astype(np.float64))
        gs.append(synth.to_bf16_bits(synth.normal_f32(61 + e, (f, d), 0.02)))
        ds.append(synth.to_bf16_bits(synth.normal_f32(71 + e, (f, d), 0.02)))
    uq, us, g, dn = map(np.stack, (ups, szs, gs, ds))
    x = synth.to_bf16_bits(synth.normal_f32(80, (T, d), 1 / 16))
    R = synth.to_bf16_bits(synth.normal_f32(81, (E, d), 0.02))
    y, idx, w, m = oracle.layer_forward(x, "bf16", R, "bf16", None, E, k, 0, True, uq, us, g, dn,
                                        "bf16", np.float32([np.inf] * E), dense=True)
    assert np.all(m == 1)       # the dense path ignores the thresholds
    X = _bits_to_f64(x, "bf16")
    ref = np.zeros((T, d))
    for t in range(T):
        for s in range(k):
            e = idx[t, s]
            # these weights are exact in bf16 (s=2^-7, z in halves), so
            # bf16_rne(dequant) is the original weight
            hg = X[t] @ _bits_to_f64(g[e], "bf16").T
            hu = X[t] @ ws[e].T
            ref[t] += w[t, s] * ((hg * expit(hg) * hu) @ _bits_to_f64(dn[e], "bf16"))
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-14)


def test_layer_dense_path_fp16_rounds_up_weights_to_fp16():
    """fp16 layers: the dense path's up weights are the dequantised INT2 weights
    rounded once to fp16 (numpy's float64 -> float16 conversion is round to
    nearest even), and the layer is the textbook SwiGLU on them.  The weights
    here are not exact in either 16-bit type, and rounding them to bf16
    instead would miss the tolerance."""
    d, f, E, k, T = 128, 64, 3, 2, 4
    uq, us, g, dn = [], [], [], []
    for e in range(E):
        w = synth.normal_f32(90 + e, (f, d), 0.02)
        q, sz = oracle.pack_up_int2(w)
        uq.append(q); us.append(sz)
        g.append(synth.to_f16_bits(synth.normal_f32(93 + e, (f, d), 0.02)))
        dn.append(synth.to_f16_bits(synth.normal_f32(96 + e, (f, d), 0.02)))
    uq, us, g, dn = map(np.stack, (uq, us, g, dn))
    x = synth.to_f16_bits(synth.normal_f32(99, (T, d), 1 / 16))
    R = synth.to_f16_bits(synth.normal_f32(100, (E, d), 0.02))
    y, idx, w, m = oracle.layer_forward(x, "f16", R, "f16", None, E, k, 0, True, uq, us, g, dn,
                                        "f16", np.float32([np.inf] * E), dense=True)
    assert np.all(m == 1)
    X = _bits_to_f64(x, "f16")

    def swiglu(t, e, up):
        hg = X[t] @ _bits_to_f64(g[e], "f16").T
        hu = X[t] @ up.T
        return (hg * expit(hg) * hu) @ _bits_to_f64(dn[e], "f16")

    ref = np.zeros((T, d))
    ref_bf = np.zeros((T, d))
    for t in range(T):
        for s in range(k):
            e = idx[t, s]
            wq = oracle.dequant_up(uq[e], us[e], d)                     # exact, float64
            ref[t] += w[t, s] * swiglu(t, e, wq.astype(np.float16).astype(np.float64))
            ref_bf[t] += w[t, s] * swiglu(t, e, _bits_to_f64(synth.to_bf16_bits(wq), "bf16"))
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-14)
    assert np.abs(ref_bf - ref).max() > 1e-6 * np.abs(ref).max()


def test_layer_fed_topk_and_masks():
    d, f, E, k, S, T = 64, 64, 5, 2, 1, 4
    uq, us, g, dn = _tiny_layer(90, d, f, E, S)
    x, R = _router_case(91, T, d, E)
    thr = np.float32([0.01] * (E + S))
    y, idx, w, m = oracle.layer_forward(x, "f16", R, "f16", None, E, k, S, True, uq, us, g, dn,
                                        "f16", thr)
    y2, idx2, w2, m2 = oracle.layer_forward(x, "f16", R, "f16", None, E, k, S, True, uq, us, g, dn,
                                            "f16", thr, topk_in=idx, masks_in=m)
    np.testing.assert_array_equal(idx2, idx)
    np.testing.assert_array_equal(m2, m)
    np.testing.assert_allclose(w2, w, rtol=1e-15)
    np.testing.assert_allclose(y2, y, rtol=1e-15, atol=0)
    # feeding a reversed choice changes the weights consistently
    rev = idx[:, ::-1].copy()
    _, idx3, w3, _ = oracle.layer_forward(x, "f16", R, "f16", None, E, k, S, True, uq, us, g, dn,
                                          "f16", thr, topk_in=rev)
    np.testing.assert_allclose(w3, w[:, ::-1], rtol=1e-14)


# Closed forms of the linear-interpolation quantile (the threshold calibration
# reading): for sorted values x_(0) <= ... <= x_(n-1) and h = q (n - 1), the
# quantile is x_(floor h) + (h - floor h) (x_(floor h + 1) - x_(floor h)).  Each
# expected value below is worked out by hand; the cases are chosen so that a
# swapped q (q <-> 1 - q), another interpolation rule (lower, higher, nearest,
# midpoint) or an off-by-one order statistic gives a different number.
@pytest.mark.parametrize("vals,q,want", [
    (np.arange(11.0), 0.9, 9.0),                    # h = 9 exactly
    (np.arange(0.0, 50.0, 10.0), 0.8, 32.0),        # h = 3.2: 30 + 0.2 * 10 (lower 30, midpoint 35)
    (np.arange(0.0, 50.0, 10.0), 0.2, 8.0),         # h = 0.8: 0 + 0.8 * 10 (swapped q gives 32)
    (np.array([16.0, 1.0, 8.0, 2.0, 4.0]), 0.3, 2.4),   # unsorted; h = 1.2: 2 + 0.2 * 2
    (np.array([16.0, 1.0, 8.0, 2.0, 4.0]), 0.7, 7.2),   # h = 2.8: 4 + 0.8 * 4
    (np.array([5.0, 1.0, 5.0, 3.0, 5.0, 0.0]), 0.5, 4.0),   # ties; h = 2.5: 3 + 0.5 * 2
    (np.array([5.0, 1.0, 5.0, 3.0, 5.0, 0.0]), 0.1, 0.5),   # h = 0.5: 0 + 0.5 * 1
    (np.array([5.0, 1.0, 5.0, 3.0, 5.0, 0.0]), 0.95, 5.0),  # h = 4.75 between equal values
    (np.array([5.0, 1.0, 5.0, 3.0, 5.0, 0.0]), 1.0, 5.0),   # q = 1: the largest
    (np.array([5.0, 1.0, 5.0, 3.0, 5.0, 0.0]), 0.0, 0.0),   # q = 0: the smallest
    (np.array([0.25]), 0.37, 0.25),                  # one value
    (np.arange(1001.0) * 0.5, 0.9, 450.0),          # h = 900: the 901st value, 900 * 0.5
    (np.arange(1001.0) * 0.5, 0.1234, 61.7),        # h = 123.4: 61.5 + 0.4 * 0.5
])
def test_calibrate_threshold_closed_forms(vals, q, want):
    t = oracle.calibrate_threshold(vals, q)
    assert t.dtype == np.float32
    assert t == np.float32(want), (t, want)


def test_calibrate_threshold_order_statistics_brute_force():
    """At every q = i / (n - 1) the quantile is the i-th smallest value itself,
    found here by counting (no sort): the value with exactly i values below it."""
    rng = np.random.default_rng(5)
    n = 41
    vals = rng.permutation(np.arange(n) * 0.75 + 0.125)        # distinct, exact in fp32
    for i in range(n):
        below = np.array([(vals < v).sum() for v in vals])
        want = vals[below == i][0]
        assert oracle.calibrate_threshold(vals, i / (n - 1)) == np.float32(want)


def test_calibrated_threshold_realises_sparsity():
    d, f = 256, 704
    _, up_q, up_sz, gb, db = _tiny_expert(100, d, f)
    xc = synth.to_f16_bits(synth.calibration_f32(1, d, 1 / 16))
    v, _, _ = oracle.expert_forward(xc, "f16", up_q, up_sz, gb, db, "f16", thr=np.inf)
    t50 = oracle.calibrate_threshold(np.abs(v), 0.5)
    _, m, _ = oracle.expert_forward(xc, "f16", up_q, up_sz, gb, db, "f16", thr=t50)
    assert abs(1 - m.mean() - 0.5) < 0.01


# ------------------------------------------------------------------ EAM / EAMC
# MoE-Infinity review, "4.3" (EAM: tokens routed to each of the L x E experts;
# the request-level EAM adds up the iterations) and "4.5" (nearest past EAM by
# cosine distance of the flattened matrices).

def test_ream_add_is_bincount_of_routed_experts():
    rng = np.random.default_rng(41)
    L, E, k, T = 4, 8, 2, 37
    ream = rng.integers(0, 50, size=(L, E)).astype(np.int32)
    want = ream.astype(np.int64).copy()
    for layer in (0, 3, 3, 1):
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        cnt = np.bincount(idx.ravel(), minlength=E).astype(np.int32)
        oracle.ream_add(ream, layer, cnt)
        want[layer] += cnt
        assert cnt.sum() == T * k
    np.testing.assert_array_equal(ream, want)


def test_ream_add_from_router_counts():
    # the count the oracle's router reports is the routed tokens per expert
    rng = np.random.default_rng(42)
    T, d, E, k = 9, 64, 6, 2
    x = oracle_f32_bits(rng.standard_normal((T, d)))
    R = oracle_f32_bits(rng.standard_normal((E, d)) * 0.1)
    r = oracle.route_topk(x, "f32", R, "f32", E, k)
    idx, cnt = r["topk_idx"], r["expert_count"]
    ream = np.zeros((3, E), dtype=np.int32)
    oracle.ream_add(ream, 2, cnt)
    np.testing.assert_array_equal(ream[2], np.bincount(idx.ravel(), minlength=E))
    assert ream[:2].sum() == 0


def oracle_f32_bits(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def test_eamc_distance_matches_scipy_cosine():
    from scipy.spatial.distance import cosine
    rng = np.random.default_rng(43)
    for n, ln in ((1, 7), (13, 256), (40, 1728)):
        b = rng.integers(0, 300, size=(n, ln)).astype(np.int32)
        b[:, rng.random(ln) < 0.5] = 0                    # sparse activation
        q = rng.integers(0, 300, size=ln).astype(np.int32)
        i, dist = oracle.eamc_match(b, q)
        ref = np.array([cosine(q.astype(np.float64), r.astype(np.float64)) for r in b])
        np.testing.assert_allclose(dist, ref, rtol=0, atol=1e-13)
        assert i == int(np.argmin(ref))


def test_eamc_closed_forms():
    q = np.array([3, 0, 4, 0], dtype=np.int32)
    b = np.array([[3, 0, 4, 0],          # same: 0
                  [6, 0, 8, 0],          # same direction: 0
                  [0, 5, 0, 0],          # orthogonal: 1
                  [0, 0, 0, 0],          # zero vector: 1
                  [3, 4, 0, 0],          # cos = 9/25
                  [1, 0, 0, 0]],         # cos = 3/5
                 dtype=np.int32)
    i, dist = oracle.eamc_match(b, q)
    assert abs(dist[0]) < 1e-15 and abs(dist[1]) < 1e-15
    assert dist[2] == 1.0 and dist[3] == 1.0
    assert abs(dist[4] - (1 - 9 / 25)) < 1e-15
    assert abs(dist[5] - (1 - 3 / 5)) < 1e-15
    assert i in (0, 1) and dist[i] == dist[:2].min()
    i, dist = oracle.eamc_match(b, np.zeros(4, dtype=np.int32))
    assert i == 0 and np.all(dist == 1.0)                 # all equal: lowest index


def test_eamc_argmin_bruteforce_ties_and_invalid():
    rng = np.random.default_rng(44)
    for trial in range(30):
        n, ln = int(rng.integers(1, 12)), int(rng.integers(1, 9))
        b = rng.integers(0, 4, size=(n, ln)).astype(np.int32)
        b[rng.integers(0, n)] = b[rng.integers(0, n)]       # a duplicate: exact tie
        q = rng.integers(0, 4, size=ln).astype(np.int32)
        if trial % 5 == 0:
            b[rng.integers(0, n), rng.integers(0, ln)] = 1 << 22    # out of range
        if trial % 7 == 0:
            b[rng.integers(0, n), rng.integers(0, ln)] = -1
        i, dist = oracle.eamc_match(b, q)
        best, bd = -1, None
        for r in range(n):
            row = [int(v) for v in b[r]]
            if any(v < 0 or v >= 1 << 22 for v in row):
                assert math.isnan(dist[r])
                continue
            qq = [int(v) for v in q]
            ab = sum(x * y for x, y in zip(qq, row))
            aa = sum(x * x for x in qq)
            bb = sum(y * y for y in row)
            dd = 1.0 if aa == 0 or bb == 0 else 1.0 - ab / math.sqrt(aa * bb)
            assert abs(dist[r] - dd) < 1e-15
            if best < 0 or dd < bd:
                best, bd = r, dd
        assert i == best
    b = np.ones((3, 4), dtype=np.int32)
    q = np.array([1, 2, 3, 1 << 22], dtype=np.int32)
    i, dist = oracle.eamc_match(b, q)
    assert i == -1 and np.all(np.isnan(dist))


# ------------------------------------------------------------------ other up widths
# FloE review, "敏感度分析": the up projection quantised to 8, 4 and 1 bits as
# well as 2; the same group-64 min-max scheme with 2^bits - 1 levels.

def unpack_plain(up_q, d, bits):
    """Codes [f][d] from rows that hold input k at bit k*bits (LSB first)."""
    b = np.unpackbits(np.ascontiguousarray(up_q), axis=1, bitorder="little").astype(np.int64)
    b = b.reshape(up_q.shape[0], d, bits)
    return (b << np.arange(bits)).sum(-1)


def exact_bits_expert(rng, d, f, bits, s_pow=-9):
    L = (1 << bits) - 1
    G = d // 64
    q = rng.integers(0, L + 1, size=(f, d))
    q[:, ::64] = 0
    q[:, 1::64] = L
    z = rng.integers(0, L + 1, size=(f, G)).astype(np.float64)   # integer zeros: exact
    if bits == 1:
        z[:] = 0.0
    s = 2.0 ** s_pow
    w = s * (q - np.repeat(z, 64, axis=1))
    w32 = w.astype(np.float32)
    assert np.all(w32.astype(np.float64) == w)
    return w32, q, s, z


@pytest.mark.parametrize("bits", [1, 4, 8])
def test_pack_bits_exact_round_trip_and_layout(bits):
    rng = np.random.default_rng(70 + bits)
    d, f = 256, 7
    w, q, s, z = exact_bits_expert(rng, d, f, bits)
    up_q, up_sz = oracle.pack_up_bits(w, bits)
    assert up_q.shape == (f, d * bits // 8)
    assert np.all(up_sz[..., 0] == bits16(f16(np.full((f, d // 64), s))))
    zb = up_sz[..., 1]
    assert np.all((zb == bits16(f16(z))) | ((z == 0) & np.isin(zb, (0, 0x8000))))
    assert np.array_equal(unpack_plain(up_q, d, bits), q)
    assert np.array_equal(oracle.dequant_up_bits(up_q, up_sz, d, bits), w.astype(np.float64))


def test_pack_bits_single_code_positions():
    d = 64
    for bits in (1, 4, 8):
        L = (1 << bits) - 1
        for k in (0, 1, 5, 33, 63):
            w = np.zeros((1, d), dtype=np.float32)
            w[0, k] = float(L)          # min 0, max L -> s = 1, z = 0, code L at k
            up_q, _ = oracle.pack_up_bits(w, bits)
            bit = k * bits
            expect = np.zeros(d * bits // 8, dtype=np.uint8)
            expect[bit // 8] = L << (bit % 8)
            assert np.array_equal(up_q[0], expect), (bits, k)


@pytest.mark.parametrize("bits", [1, 4, 8])
def test_pack_bits_error_bound(bits):
    w = synth.normal_f32(5000 + bits, (32, 512), 0.02)
    up_q, up_sz = oracle.pack_up_bits(w, bits)
    deq = oracle.dequant_up_bits(up_q, up_sz, 512, bits)
    s = np.repeat(np.asarray([[oracle.half_to_double(b) for b in row] for row in up_sz[..., 0]]), 64, 1)
    z = np.repeat(np.asarray([[oracle.half_to_double(b) for b in row] for row in up_sz[..., 1]]), 64, 1)
    err = np.abs(deq - w.astype(np.float64))
    L = (1 << bits) - 1
    # half a step, plus the fp16 rounding of z (< 2^-11 relative, times s)
    assert np.all(err <= 0.5 * s + np.abs(z) * s * 2.0 ** -10 + 1e-12)
    # more bits, smaller error
    if bits > 1:
        lo_q, lo_sz = oracle.pack_up_bits(w, 1 if bits == 4 else 4)
        lo = oracle.dequant_up_bits(lo_q, lo_sz, 512, 1 if bits == 4 else 4)
        assert np.abs(deq - w).mean() < np.abs(lo - w).mean()
    codes = unpack_plain(up_q, 512, bits).reshape(32, 8, 64)
    g = w.reshape(32, 8, 64)
    assert np.all(np.take_along_axis(codes, g.argmin(-1)[..., None], -1) == 0)
    assert np.all(np.take_along_axis(codes, g.argmax(-1)[..., None], -1) == L)


def test_pack_bits_two_is_the_int2_format():
    w = synth.normal_f32(5100, (16, 256), 0.02)
    a = oracle.pack_up_bits(w, 2)
    b = oracle.pack_up_int2(w)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("bits", [1, 4, 8])
def test_expert_bits_dense_threshold_is_textbook_swiglu(bits):
    d, f, T = 256, 128, 2
    rng = np.random.default_rng(80 + bits)
    w_up, _, _, _ = exact_bits_expert(rng, d, f, bits)
    up_q, up_sz = oracle.pack_up_bits(w_up, bits)
    gb = synth.to_bits(synth.normal_f32(81, (f, d), 0.02), "f16")
    db = synth.to_bits(synth.normal_f32(82, (f, d), 0.02), "f16")
    x = synth.to_bits(synth.normal_f32(83, (T, d), 1 / 16), "f16")
    v, m, y = oracle.expert_forward(x, "f16", up_q, up_sz, gb, db, "f16", thr=-1.0, bits=bits)
    X = _bits_to_f64(x, "f16")
    Wg = _bits_to_f64(gb, "f16").T
    Wd = _bits_to_f64(db, "f16")
    Wu = w_up.astype(np.float64).T
    ref = (X @ Wg * expit(X @ Wg) * (X @ Wu)) @ Wd
    assert np.all(m == 1)
    np.testing.assert_allclose(v, X @ Wu, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-14)
    # a threshold keeps exactly the channels with |v| > t
    t = float(np.median(np.abs(v)))
    v2, m2, _ = oracle.expert_forward(x, "f16", up_q, up_sz, gb, db, "f16", thr=t, bits=bits)
    assert np.array_equal(m2, (np.abs(v2) > np.float32(t)).astype(np.uint8))


# ------------------------------------------------------------------ input recipe
# FloE review, "双稀疏预测器", observation 3: the hidden states of consecutive
# MoE layers have cosine similarity above 0.95.  The 32-layer stack's hidden
# stream is built to respect that; this holds it to it, in fp32 and after the
# fp16 cast the layers are fed.

def test_stack_hidden_stream_keeps_cosine_above_095():
    c = synth.CONFIGS[synth.CFG_STACK]
    for T in (1, 16):
        xs = synth.hidden_stream_f32(synth.CFG_STACK, c["L"], T, c["d"], c["x_scale"])
        for arr in (xs.astype(np.float64),
                    synth.to_f16_bits(xs).view(np.float16).astype(np.float64)):
            a, b = arr[:-1], arr[1:]
            cos = (a * b).sum(-1) / (np.linalg.norm(a, axis=-1) * np.linalg.norm(b, axis=-1))
            assert cos.shape == (c["L"] - 1, T)
            assert cos.min() >= 0.95, cos.min()


def test_layer_per_expert_dense_flags_pick_each_experts_path():
    """dense_experts: the flagged experts take the dense path (every channel,
    up weights rounded to the layer type) and the others Algorithm 1; the
    layer is the weighted sum of those per-expert results, each computed
    alone."""
    d, f, E, k, S, T = 128, 64, 4, 2, 1, 5
    uq, us, g, dn = _tiny_layer(93, d, f, E, S)
    x, R = _router_case(94, T, d, E)
    thr = np.float32([0.01] * (E + S))
    flags = np.array([1, 0, 1, 0, 1], dtype=np.uint8)
    y, idx, w, m = oracle.layer_forward(x, "f16", R, "f16", None, E, k, S, True, uq, us, g, dn,
                                        "f16", thr, dense_experts=flags)
    y_dense, _, _, _ = oracle.layer_forward(x, "f16", R, "f16", None, E, k, S, True, uq, us, g,
                                            dn, "f16", thr, dense=True)
    y_sparse, _, _, _ = oracle.layer_forward(x, "f16", R, "f16", None, E, k, S, True, uq, us, g,
                                             dn, "f16", thr)
    ref = np.zeros((T, d))
    for t in range(T):
        for s_ in range(k + S):
            e = idx[t, s_] if s_ < k else E + s_ - k
            sc = w[t, s_] if s_ < k else 1.0
            one_hot = np.zeros(E + S, np.uint8)
            one_hot[e] = 1
            # the expert alone through a layer call with only it flagged or not
            if flags[e]:
                assert np.all(m[t, s_] == 1)
                up16 = oracle.dequant_up(uq[e], us[e], d).astype(np.float16).astype(np.float64)
                X = _bits_to_f64(x[t:t + 1], "f16")
                hg = X @ _bits_to_f64(g[e], "f16").T
                hu = X @ up16.T
                ref[t] += sc * ((hg * expit(hg) * hu) @ _bits_to_f64(dn[e], "f16"))[0]
            else:
                _, _, ye = oracle.expert_forward(x[t:t + 1], "f16", uq[e], us[e], g[e], dn[e],
                                                 "f16", thr[e])
                ref[t] += sc * ye[0]
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-14)
    assert not np.allclose(y, y_dense) and not np.allclose(y, y_sparse)
