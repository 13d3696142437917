"""Pins for the layer-scaffold oracle (conv along paths, history, gating) and
the speculative-step == autoregressive-decode property of the whole stack."""

import numpy as np

from linear_attention_gdn_amd import workloads as W
from oracle import layer as LY


def _causal_conv(x, w):
    """Per-channel causal conv via np.convolve: y[t] = sum_i w[i] x[t-i]."""
    T, C = x.shape
    return np.stack([np.convolve(x[:, c], w[c])[:T] for c in range(C)], axis=1)


def test_tree_conv_on_a_chain_is_causal_convolution():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((9, 5))
    w = rng.standard_normal((5, LY.CONV_TAPS))
    hist = np.zeros((LY.CONV_TAPS - 1, 5))
    y = LY.tree_conv(x, W.chain_parents(9), w, hist)
    np.testing.assert_allclose(y, _causal_conv(x, w), atol=1e-13)


def test_history_continues_the_sequence():
    rng = np.random.default_rng(1)
    seq = rng.standard_normal((12, 4))
    w = rng.standard_normal((4, LY.CONV_TAPS))
    full = _causal_conv(seq, w)
    hist = seq[8:5:-1]  # tokens 8, 7, 6: most recent first
    y = LY.tree_conv(seq[9:], W.chain_parents(3), w, hist)
    np.testing.assert_allclose(y, full[9:], atol=1e-13)


def test_tree_conv_follows_root_paths():
    rng = np.random.default_rng(2)
    par = W.random_parents(14, rng)
    x = rng.standard_normal((14, 3))
    w = rng.standard_normal((3, LY.CONV_TAPS))
    hist = rng.standard_normal((LY.CONV_TAPS - 1, 3))
    y = LY.tree_conv(x, par, w, hist)
    for t in range(14):
        path = W.root_path(par, t)
        seq = np.concatenate([hist[::-1], x[path]])
        np.testing.assert_allclose(y[t], _causal_conv(seq, w)[-1], atol=1e-13)


def test_commit_history_shifts_in_the_accepted_path():
    rng = np.random.default_rng(3)
    par = np.array([-1, 0, 1, 1, 3], np.int32)
    x = rng.standard_normal((5, 2))
    hist = rng.standard_normal((3, 2))
    np.testing.assert_array_equal(LY.commit_history(x, par, hist, -1), hist)
    np.testing.assert_array_equal(LY.commit_history(x, par, hist, 0), np.stack([x[0], hist[0], hist[1]]))
    np.testing.assert_array_equal(LY.commit_history(x, par, hist, 4), np.stack([x[4], x[3], x[1]]))


def test_prep_normalises_and_maps_gates():
    rng = np.random.default_rng(4)
    H, d, N = 2, 4, 3
    C_in = 4 * H * d + 2 * H
    P = rng.standard_normal((N, C_in))
    w = rng.standard_normal((3 * H * d, LY.CONV_TAPS))
    q, k, v, beta, g, gate = LY.layer_prep(P, W.chain_parents(N), w, np.zeros((3, 3 * H * d)),
                                           H, d, d, gate_shift=2.0)
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 1.0, atol=1e-14)
    np.testing.assert_allclose(np.linalg.norm(k, axis=-1), 1.0, atol=1e-14)
    a = P[:, 4 * H * d:4 * H * d + H]
    bl = P[:, 4 * H * d + H:]
    np.testing.assert_allclose(beta, 1 / (1 + np.exp(-bl)), rtol=1e-14)
    np.testing.assert_allclose(np.exp(g), 1 / (1 + np.exp(a + 2.0)), rtol=1e-12)
    np.testing.assert_array_equal(gate, P[:, 3 * H * d:4 * H * d])


def _toy_stack(seed, L=3, D=24, H=2, d=8):
    rng = np.random.default_rng(seed)
    C_in = 4 * H * d + 2 * H
    wt = LY.StackWeights([rng.standard_normal((C_in, D)) / np.sqrt(D) for _ in range(L)],
                         [rng.standard_normal((3 * H * d, LY.CONV_TAPS)) / 2 for _ in range(L)],
                         [rng.standard_normal((D, H * d)) / np.sqrt(H * d) for _ in range(L)],
                         H, d, d)
    states = [0.05 * rng.standard_normal((H, d, d)) for _ in range(L)]
    hists = [0.5 * rng.standard_normal((3, 3 * H * d)) for _ in range(L)]
    return wt, states, hists, rng


def test_spec_step_on_a_chain_equals_autoregressive_decode():
    """The review's exactness check (outputs match autoregressive decoding):
    a chain draft verified in one step, then committed, gives the same
    per-token outputs and the same states/histories as token-by-token decode."""
    wt, states, hists, rng = _toy_stack(5)
    N = 6
    x0 = rng.standard_normal((N, 24))
    par = W.chain_parents(N)
    x_spec, per_layer = LY.stack_spec_step(wt, x0, par, states, hists)
    last = 3
    S_spec, h_spec = LY.stack_commit(wt, par, states, hists, per_layer, last)
    S_ar, h_ar = [s.copy() for s in states], [h.copy() for h in hists]
    for t in range(last + 1):
        one = W.chain_parents(1)
        x_tok, pl = LY.stack_spec_step(wt, x0[t:t + 1], one, S_ar, h_ar)
        np.testing.assert_allclose(x_tok[0], x_spec[t], rtol=1e-10, atol=1e-12)
        S_ar, h_ar = LY.stack_commit(wt, one, S_ar, h_ar, pl, 0)
    for layer in range(wt.layers):
        np.testing.assert_allclose(S_spec[layer], S_ar[layer], rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(h_spec[layer], h_ar[layer], rtol=1e-12, atol=1e-13)


def test_spec_step_on_a_tree_matches_each_path_decoded_alone():
    wt, states, hists, rng = _toy_stack(6)
    par = np.array([-1, 0, 0, 1, 2, 4], np.int32)
    x0 = rng.standard_normal((6, 24))
    x_spec, _ = LY.stack_spec_step(wt, x0, par, states, hists)
    for t in range(6):
        path = W.root_path(par, t)
        x_path, _ = LY.stack_spec_step(wt, x0[path], W.chain_parents(len(path)), states, hists)
        np.testing.assert_allclose(x_path[-1], x_spec[t], rtol=1e-10, atol=1e-12)


def test_round_bf16_ties_and_cases():
    r = LY.round_bf16
    assert r(1.0) == 1.0
    assert r(1 + 2.0 ** -8) == 1.0                      # tie -> even (mantissa 0)
    assert r(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6        # tie -> even (mantissa 2)
    assert r(1 + 2.0 ** -8 + 2.0 ** -20) == 1 + 2.0 ** -7  # above the tie
    assert r(-(1 + 3 * 2.0 ** -8)) == -(1 + 2.0 ** -6)
    assert r(0.0) == 0.0
    assert r(3.0 * 2.0 ** -130) == 3.0 * 2.0 ** -130    # few bits: exact
    assert r(255.5) == 256.0 and r(254.5) == 254.0      # spacing 1 in [128, 256)


def test_round_bf16_matches_float32_bit_rounding():
    """Against the generator's independent rule (RNE on float32 bit patterns)."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    ref = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x)).astype(np.float64)
    np.testing.assert_array_equal(LY.round_bf16(x.astype(np.float64)), ref)


# ---------------------------------------------------------------------------
# the activation: SiLU(x) = x sigmoid(x), pinned by closed forms
# ---------------------------------------------------------------------------

LN3 = np.log(3.0)  # sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4 exactly


def test_silu_closed_forms():
    """SiLU is odd up to the identity (silu(x) - silu(-x) = x), vanishes at 0,
    tends to x for large x and to 0 for very negative x, and is known in
    closed form at +-ln 3.  A logistic sigmoid in its place fails every line."""
    s = LY.silu
    assert s(0.0) == 0.0
    x = np.linspace(-6.0, 6.0, 49)
    np.testing.assert_allclose(s(x) - s(-x), x, rtol=0, atol=1e-14)
    assert abs(s(30.0) - 30.0) < 1e-10 and abs(s(40.0) - 40.0) < 1e-14
    assert abs(s(-40.0)) < 1e-15
    np.testing.assert_allclose(s(np.array([LN3, -LN3])), [0.75 * LN3, -0.25 * LN3],
                               rtol=1e-15)
    # minimum of x sigmoid(x): at x* with 1 + x*(1 - sigmoid(x*)) = 0, x* = -1.27846...
    xs = np.linspace(-1.4, -1.15, 25001)
    assert abs(xs[np.argmin(s(xs))] + 1.2784645) < 2e-5


def test_gate_merge_closed_forms():
    """o * SiLU(gate): zero gate closes the output, a large gate passes it,
    and gate = +-ln 3 scales it by 3/4 ln 3 and -1/4 ln 3."""
    rng = np.random.default_rng(11)
    o = rng.standard_normal((3, 2, 4))
    flat = o.reshape(3, 8)
    np.testing.assert_array_equal(LY.gate_merge(o, np.zeros((3, 8))), np.zeros((3, 8)))
    np.testing.assert_allclose(LY.gate_merge(o, np.full((3, 8), 40.0)), 40.0 * flat, rtol=1e-15)
    gate = np.where(np.arange(8) % 2 == 0, LN3, -LN3)[None, :].repeat(3, 0)
    want = flat * np.where(np.arange(8) % 2 == 0, 0.75 * LN3, -0.25 * LN3)
    np.testing.assert_allclose(LY.gate_merge(o, gate), want, rtol=1e-14)


def test_prep_applies_silu_after_the_path_convolution():
    """A 2-node chain with all-ones taps: node 1's convolution input is
    node 1, node 0, then the two most recent history rows.  The channel sums
    are chosen to be +-ln 3 (and 0), so the activation's output is known in
    closed form: v = SiLU(c) and q, k are SiLU(c) normalised per head."""
    H, d = 1, 2
    Cc = 3 * H * d
    w = np.ones((Cc, LY.CONV_TAPS))
    # per channel: (node 0, node 1, hist row 0, hist row 1); node 1's sum =
    # x1 + x0 + h0 + h1, node 0's sum = x0 + h0 + h1 + h2
    P = np.zeros((2, 4 * H * d + 2 * H))
    hist = np.zeros((3, Cc))
    sums = np.array([LN3, -LN3, -LN3, LN3, LN3, 0.0])  # q^ (2), k^ (2), v^ (2) at node 1
    P[1, :Cc] = sums / 2
    P[0, :Cc] = sums / 4
    hist[0] = sums / 8
    hist[1] = sums / 8
    q, k, v, beta, g, _ = LY.layer_prep(P, W.chain_parents(2), w, hist, H, d, d)
    np.testing.assert_allclose(v[1, 0], [0.75 * LN3, 0.0], rtol=1e-15, atol=1e-16)
    # SiLU(+-ln 3) = (3/4, -1/4) ln 3, so the normalised rows are (3, -1)/sqrt(10)
    np.testing.assert_allclose(q[1, 0], np.array([3.0, -1.0]) / np.sqrt(10.0), rtol=1e-14)
    np.testing.assert_allclose(k[1, 0], np.array([-1.0, 3.0]) / np.sqrt(10.0), rtol=1e-14)
    # node 0: history rows 0..2 and node 0 itself: sums/4 + sums/8 + sums/8 + 0
    np.testing.assert_allclose(v[0, 0], [0.5 * LN3 / (1 + 3.0 ** -0.5), 0.0], rtol=1e-14,
                               atol=1e-16)
