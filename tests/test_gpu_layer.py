"""GPU parity of the layer scaffold (include/gdnlayer.h) against the oracle in
oracle/layer.py, through the C ABI, on seeded inputs: each stage alone, one
speculative step of the full 24-layer stack at its real sizes, and the
chain-verify == token-by-token decode property of the stack on the GPU."""

import numpy as np
import pytest
import torch

from linear_attention_gdn_amd import gdnspec as G
from linear_attention_gdn_amd import workloads as W
from linear_attention_gdn_amd.stack import GdnStack
from oracle import layer as LY
from oracle import oracle as O

from _gpu import TOL_OUT, TOL_STATE, dev_tensors, slice_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda"
U_BF16 = 2.0 ** -8  # bf16 rounding: |round(x) - x| <= 2^-8 |x|

# Parity of the stack is gated layer by layer: each GPU layer gets the
# oracle's own input rows of that layer (data flows from the oracle to the GPU
# only), so every layer sees what layer 0 sees in a free-running run, and is
# held to the verifier's bounds (test_stack_layerwise_*).
#
# Free-running (each side feeding its own layer outputs forward) is a drift
# report, not a parity gate.  Stacked layers re-round every layer's inputs to
# bf16; two correct implementations that differ only in FP32-vs-FP64 rounding
# then round some inputs one bf16 step apart, each such flip moves every
# projection output of its node slightly, and later layers flip more inputs:
# past the first layer the two agree to a few bf16 units.  The oracle shows the
# same spread against itself when its values are perturbed by 2^-24 before
# rounding (24 layers, six perturbations: state max error up to 1.3e-2 = 3.3
# units, RMS up to 4.9e-3 = 1.25 units).  The drift checks below only guard
# against gross breakage (8 units max, 2 units RMS per head); they are also the
# bounds of the GPU-against-GPU equivalence of chain verification and
# token-by-token decoding, whose two routes round their own layer inputs.
DRIFT_STATE_MAX = 8 * U_BF16
DRIFT_STATE_RMS = 2 * U_BF16


def bf(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).to(DEV).view(
        torch.bfloat16)


def f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(DEV)


def i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(DEV)


def wide(bits):
    return W.bf16_bits_to_f32(bits).astype(np.float64)


def bits_of(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def rel(gpu, ref):
    return np.abs(np.asarray(gpu, np.float64) - ref).max() / np.abs(ref).max()


def assert_bf16_close(gpu_bits, ref, slack):
    """Each bf16 value is within one rounding of the exact value, plus `slack`
    (relative to the largest |ref|) for the FP32 arithmetic before rounding."""
    g = wide(gpu_bits)
    bound = U_BF16 * np.abs(ref) + slack * np.abs(ref).max()
    bad = np.abs(g - ref) > bound
    assert not bad.any(), f"{bad.sum()} values off; worst {np.abs(g - ref).max():.3e}"


# ---------------------------------------------------------------------------
# gdn_linear
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,Nc,K", [(1, 16, 512), (5, 48, 512), (16, 64, 1024), (33, 80, 256),
                                    (64, 32, 1536), (32, 2048, 2048), (32, 8192, 2048),
                                    (1, 8192, 2048), (7, 8208, 2048), (40, 96, 4096)])
@pytest.mark.parametrize("resid", [False, True])
def test_linear_matches_oracle(M, Nc, K, resid):
    """Both weight layouts, every kernel form (all-in-flight for K = 256,
    512, 1024, 2048; the pipelined loop for 1536 and 4096), ragged M and Nc."""
    rng = np.random.default_rng(M * 100003 + Nc * 7 + K + resid)
    A = W.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    Wt = W.f32_to_bf16_bits(rng.standard_normal((Nc, K), dtype=np.float32) * np.float32(K ** -0.5))
    R = rng.standard_normal((M, Nc)).astype(np.float32) if resid else None
    ref = LY.linear(wide(A), wide(Wt), resid=R)
    Wd = bf(Wt)
    Wp = torch.empty_like(Wd)
    G.gdn_pack_weights(Wd, Wp)
    outs = []
    for Wx, layout in ((Wd, G.GDN_W_ROWS), (Wp, G.GDN_W_PACKED)):
        C = torch.full((M, Nc), float("nan"), device=DEV)
        Cb = torch.empty((M, Nc), dtype=torch.bfloat16, device=DEV)
        G.gdn_linear(bf(A), Wx, C=C, R=f32(R) if resid else None, C_bf16=Cb, w_layout=layout)
        outs.append((C, Cb))
    torch.cuda.synchronize()
    c = outs[0][0].cpu().numpy()
    assert rel(c, ref) <= 1e-5
    # the bf16 copy is C rounded to nearest even
    np.testing.assert_array_equal(bits_of(outs[0][1]), W.f32_to_bf16_bits(c))
    assert_bf16_close(bits_of(outs[0][1]), ref, 1e-5)
    # the packed layout gives bitwise the same results
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_pack_weights_layout():
    """Packed chunk (tile t, k-step s, lane l) holds W[16 t + l % 16][32 s + 8 (l // 16) + e]."""
    rng = np.random.default_rng(17)
    Nc, K = 48, 512
    Wt = rng.integers(0, 1 << 16, size=(Nc, K), dtype=np.uint16)
    Wp = torch.empty((Nc, K), dtype=torch.bfloat16, device=DEV)
    G.gdn_pack_weights(bf(Wt), Wp)
    torch.cuda.synchronize()
    got = bits_of(Wp).reshape(Nc // 16, K // 32, 64, 8)
    l = np.arange(64)
    for t in range(Nc // 16):
        for s_ in range(K // 32):
            want = np.stack([Wt[16 * t + l % 16, 32 * s_ + 8 * (l // 16) + e] for e in range(8)], 1)
            np.testing.assert_array_equal(got[t, s_], want)


def test_linear_in_place_residual_and_bitwise_repeat():
    rng = np.random.default_rng(5)
    M, Nc, K = 32, 2048, 2048
    A = W.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    Wt = W.f32_to_bf16_bits(rng.standard_normal((Nc, K), dtype=np.float32) * np.float32(K ** -0.5))
    R = rng.standard_normal((M, Nc)).astype(np.float32)
    ref = LY.linear(wide(A), wide(Wt), resid=R)
    X = f32(R)
    G.gdn_linear(bf(A), bf(Wt), C=X, R=X)
    Y = torch.empty_like(X)
    G.gdn_linear(bf(A), bf(Wt), C=Y, R=f32(R))
    torch.cuda.synchronize()
    assert rel(X.cpu().numpy(), ref) <= 1e-5
    assert torch.equal(X, Y)


# ---------------------------------------------------------------------------
# gdn_layer_prep
# ---------------------------------------------------------------------------

def _topology(kind, N, rng):
    return {"window": lambda: W.window_tree_parents(N, rng),
            "branching": lambda: W.branching_tree_parents(N, rng),
            "random": lambda: W.random_parents(N, rng),
            "chain": lambda: W.chain_parents(N)}[kind]()


@pytest.mark.parametrize("B,N,H,dk,dv,D,topo", [(1, 32, 8, 256, 256, 2048, "window"),
                                                (2, 64, 2, 64, 32, 72, "branching"),
                                                (2, 7, 3, 40, 24, 4104, "random"),
                                                (3, 1, 2, 16, 8, 8, "chain"),
                                                (1, 12, 1, 256, 256, 512, "chain")])
def test_layer_prep_matches_oracle(B, N, H, dk, dv, D, topo):
    rng = np.random.default_rng(B * 1000 + N * 10 + H)
    npj = 2 * H * (dk + dv)
    Cc = H * (2 * dk + dv)
    P = rng.standard_normal((B, N, npj)).astype(np.float32)
    x = W.f32_to_bf16_bits(rng.standard_normal((B, N, D), dtype=np.float32))
    W_ab = W.f32_to_bf16_bits(rng.standard_normal((2 * H, D), dtype=np.float32) *
                              np.float32(D ** -0.5))
    parents = np.stack([_topology(topo, N, rng) for _ in range(B)]).astype(np.int32)
    conv_w = (0.5 * rng.standard_normal((Cc, 4))).astype(np.float32)
    hist = rng.standard_normal((B, 3, Cc)).astype(np.float32)
    q = torch.empty((B, N, H, dk), dtype=torch.bfloat16, device=DEV)
    k = torch.empty_like(q)
    v = torch.empty((B, N, H, dv), dtype=torch.bfloat16, device=DEV)
    beta = torch.full((B, N, H), float("nan"), device=DEV)
    g = torch.full((B, N, H), float("nan"), device=DEV)
    G.gdn_layer_prep(f32(P), bf(x), bf(W_ab), i32(parents), f32(conv_w), f32(hist), q, k, v,
                     beta, g, gate_shift=2.0)
    torch.cuda.synchronize()
    for b in range(B):
        # the oracle's projection output: the given columns, then the logits x . W_ab
        P_full = np.concatenate([P[b].astype(np.float64), LY.linear(wide(x[b]), wide(W_ab))], 1)
        rq, rk, rv, rb, rg, _ = LY.layer_prep(P_full, parents[b], conv_w, hist[b], H, dk, dv, 2.0)
        assert_bf16_close(bits_of(q[b]), rq, 2e-6)
        assert_bf16_close(bits_of(k[b]), rk, 2e-6)
        assert_bf16_close(bits_of(v[b]), rv, 2e-6)
        # FP32 dot products of length D feed the logits
        np.testing.assert_allclose(beta[b].cpu().numpy(), rb, rtol=2e-5, atol=1e-6)
        np.testing.assert_allclose(g[b].cpu().numpy(), rg, rtol=2e-5, atol=1e-6)


# ---------------------------------------------------------------------------
# gdn_gate_merge, gdn_conv_commit
# ---------------------------------------------------------------------------

def test_gate_merge_matches_oracle():
    rng = np.random.default_rng(9)
    M, Cw, ldg, off = 37, 2048, 8208, 6144
    o = rng.standard_normal((M, Cw)).astype(np.float32)
    P = (2.0 * rng.standard_normal((M, ldg))).astype(np.float32)
    Pt = f32(P)
    Y = torch.empty((M, Cw), dtype=torch.bfloat16, device=DEV)
    G.gdn_gate_merge(f32(o), Pt[:, off:off + Cw], Y)
    torch.cuda.synchronize()
    ref = LY.gate_merge(o.reshape(M, 1, Cw), P[:, off:off + Cw])
    assert_bf16_close(bits_of(Y), ref, 1e-6)


def test_conv_commit_is_exact():
    rng = np.random.default_rng(13)
    B, N, Cc, ldP = 3, 20, 1000, 1100
    parents = np.stack([W.window_tree_parents(N, rng) for _ in range(B)]).astype(np.int32)
    P = rng.standard_normal((B, N, ldP)).astype(np.float32)
    hist0 = rng.standard_normal((B, 3, Cc)).astype(np.float32)
    # sequence 1's parent array fails the topology check in the last two cases
    bad_par = parents.copy()
    bad_par[1, 9] = 9
    for lasts, par in (([-1, 0, 5], parents), ([N - 1, 3, 2], parents), ([N, -2, 1], parents),
                       ([7, 11, -1], parents), ([7, 11, -1], bad_par), ([3, -1, 4], bad_par)):
        h = f32(hist0)
        st = torch.full((B,), 77, dtype=torch.int32, device=DEV)
        G.gdn_conv_commit(f32(P), i32(par), i32(lasts), h, dev_status=st)
        torch.cuda.synchronize()
        got = h.cpu().numpy()
        for b, last in enumerate(lasts):
            rejected = par is bad_par and b == 1 and last >= 0
            if last == -1 or (0 <= last < N and not rejected):
                assert int(st[b]) == G.GDN_OK
                ref = LY.commit_history(P[b][:, :Cc], parents[b], hist0[b], last)
                np.testing.assert_array_equal(got[b].astype(np.float64), ref)
            else:
                assert int(st[b]) == G.GDN_ERR_TOPOLOGY
                np.testing.assert_array_equal(got[b], hist0[b])


@pytest.mark.parametrize("B,Np,N,H,dk,dv,D,topo", [(1, 32, 32, 8, 256, 256, 2048, "window"),
                                                   (3, 9, 13, 2, 40, 24, 72, "random"),
                                                   (2, 64, 5, 1, 16, 8, 8, "branching")])
def test_layer_prep_delayed_is_conv_commit_then_prep(B, Np, N, H, dk, dv, D, topo):
    """The fused history commit: gdn_conv_commit of the previous step's path
    followed by gdn_layer_prep, bitwise (history, q, k, v, beta, g, status),
    for accepted, empty and out-of-range previous paths."""
    rng = np.random.default_rng(B * 77 + Np + N)
    npj = 2 * H * (dk + dv)
    Cc = H * (2 * dk + dv)
    P = f32(rng.standard_normal((B, N, npj)).astype(np.float32))
    P_prev = f32(rng.standard_normal((B, Np, npj)).astype(np.float32))
    x = bf(W.f32_to_bf16_bits(rng.standard_normal((B, N, D), dtype=np.float32)))
    W_ab = bf(W.f32_to_bf16_bits(rng.standard_normal((2 * H, D), dtype=np.float32) *
                                 np.float32(D ** -0.5)))
    parents = i32(np.stack([_topology(topo, N, rng) for _ in range(B)]))
    parents_prev = i32(np.stack([_topology(topo, Np, rng) for _ in range(B)]))
    conv_w = f32((0.5 * rng.standard_normal((Cc, 4))).astype(np.float32))
    hist0 = f32(rng.standard_normal((B, 3, Cc)).astype(np.float32))

    def outs():
        return (torch.empty((B, N, H, dk), dtype=torch.bfloat16, device=DEV),
                torch.empty((B, N, H, dk), dtype=torch.bfloat16, device=DEV),
                torch.empty((B, N, H, dv), dtype=torch.bfloat16, device=DEV),
                torch.full((B, N, H), float("nan"), device=DEV),
                torch.full((B, N, H), float("nan"), device=DEV))

    # the previous draft of sequence 0 with a parent array that fails the
    # topology check: its state commit is rejected, so its history stays
    pp_bad = parents_prev.clone()
    pp_bad[0, Np - 1] = Np - 1
    lasts_cases = [([-1] * B, parents_prev), ([Np - 1] * B, parents_prev),
                   ([int(rng.integers(0, Np)) for _ in range(B)], parents_prev),
                   ([Np] + [0] * (B - 1), parents_prev),  # out of range: that history stays
                   ([Np - 1] * B, pp_bad), ([0] * B, pp_bad)]
    for lasts, ppar in lasts_cases:
        lt = i32(np.array(lasts))
        # two calls
        h_a = hist0.clone()
        st_a = torch.full((B,), 77, dtype=torch.int32, device=DEV)
        G.gdn_conv_commit(P_prev, ppar, lt, h_a, dev_status=st_a)
        qa, ka, va, ba, ga = outs()
        G.gdn_layer_prep(P, x, W_ab, parents, conv_w, h_a, qa, ka, va, ba, ga, gate_shift=2.0)
        # one fused call
        h_b = torch.full_like(hist0, float("nan"))
        st_b = torch.full((B,), 77, dtype=torch.int32, device=DEV)
        qb, kb, vb, bb, gb = outs()
        G.gdn_layer_prep_delayed(P, x, W_ab, parents, conv_w, hist0, qb, kb, vb, bb, gb, P_prev,
                                 ppar, lt, h_b, gate_shift=2.0, dev_status=st_b)
        torch.cuda.synchronize()
        if ppar is pp_bad:  # rejected: sequence 0's history is the old one, with the status
            assert int(st_b[0]) == G.GDN_ERR_TOPOLOGY
            assert torch.equal(h_b[0], hist0[0])
        assert torch.equal(h_a, h_b), lasts
        assert torch.equal(st_a, st_b), lasts
        for a, b_ in ((qa, qb), (ka, kb), (va, vb)):
            assert torch.equal(a.view(torch.int16), b_.view(torch.int16)), lasts
        assert torch.equal(ba, bb) and torch.equal(ga, gb), lasts


# ---------------------------------------------------------------------------
# gdn_decode_step
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,H,dk,dv", [("bf16", 8, 256, 256), ("f32", 2, 64, 32),
                                           ("bf16", 3, 40, 24)])
def test_decode_step_matches_oracle(dtype, H, dk, dv):
    B = 2
    d = W.make_draft(B, 1, H, dk, dv, topology="chain", accept="full", dtype=dtype, seed=3)
    ref_out, _, _ = O.draft_verify(d)        # [B][1][H][dv]
    ref_S, _, _ = O.draft_commit(d)          # [B][H][dv][dk]
    t = dev_tensors(d)
    S = t["S0"].clone()
    out = torch.full((B, H, dv), float("nan"), device=DEV)
    G.gdn_decode_step(S, t["q"].view(B, H, dk), t["k"].view(B, H, dk), t["v"].view(B, H, dv),
                      t["beta"].view(B, H), t["g"].view(B, H), out, scale=d.scale)
    torch.cuda.synchronize()
    assert slice_rel_err(out.cpu().numpy()[:, :, None, :],
                         ref_out.transpose(0, 2, 1, 3)) <= TOL_OUT
    assert slice_rel_err(S.cpu().numpy(), ref_S) <= TOL_STATE


# ---------------------------------------------------------------------------
# the stack
# ---------------------------------------------------------------------------

def rms_rel_err(gpu, ref):
    """Largest per-head ||gpu - ref||_F / ||ref||_F; inputs shaped [H][...]."""
    return max(np.linalg.norm(np.asarray(gpu[h], np.float64) - ref[h]) / np.linalg.norm(ref[h])
               for h in range(ref.shape[0]))


def _stack_case(shape, B, N, seed):
    rng = np.random.default_rng(seed)
    layers = [W.stack_layer_weights(shape, rng) for _ in range(shape.layers)]
    S0 = W.stack_states(shape, B, rng)
    return rng, layers, S0


def _load(shape, layers, S0, B, N):
    st = GdnStack(shape, B=B, N=N)
    for l, (w_in, conv, w_o) in enumerate(layers):
        st.load_layer(l, w_in, conv, w_o, S0=S0[l])
    return st


def test_stack_spec_step_matches_oracle_24_layers():
    """One verify + commit step of the 24-layer stack (hidden 2048, h=8,
    d=256, a 32-node window tree) against the oracle run with bf16 rounding
    at the same points, free-running from the same seeded inputs: layer 0 and
    the final outputs at the parity bounds, deeper layers' states reported as
    drift (see DRIFT_STATE_MAX)."""
    shape = W.StackShape(layers=24)
    N = 32
    rng, layers, S0 = _stack_case(shape, 1, N, seed=21)
    parents, last = W.stack_drafts(rng, 1, N=N)
    x0 = W.stack_inputs(rng, N, shape.D)
    st = _load(shape, layers, S0, 1, N)
    st.set_inputs(f32(wide(x0)), bf(x0))
    par_t, last_t = i32(parents), i32(last)
    st.verify(par_t)
    st.commit(par_t, last_t)
    torch.cuda.synchronize()
    assert int(st.status[0]) == G.GDN_OK

    wt = LY.StackWeights([wide(w) for w, _, _ in layers], [c for _, c, _ in layers],
                         [wide(w) for _, _, w in layers], shape.H, shape.dk, shape.dv, bf16=True)
    zeros = [np.zeros((3, shape.n_conv)) for _ in range(shape.layers)]
    states = [S0[l][0].astype(np.float64) for l in range(shape.layers)]
    x_ref, per_layer = LY.stack_spec_step(wt, wide(x0), parents[0], states, zeros)
    S_ref, h_ref = LY.stack_commit(wt, parents[0], states, zeros, per_layer, int(last[0]))
    S_gpu = st.S.cpu().numpy()
    h_gpu = st.hist.cpu().numpy()
    e_x = rel(st.x.cpu().numpy(), x_ref)
    e_S = [slice_rel_err(S_gpu[l], S_ref[l][None]) for l in range(shape.layers)]
    e_R = [rms_rel_err(S_gpu[l, 0], S_ref[l]) for l in range(shape.layers)]
    e_h = [rel(h_gpu[l, 0], h_ref[l]) for l in range(shape.layers)]
    print(f"\n24-layer step: output {e_x:.2e}; layer-0 state {e_S[0]:.2e}; states max "
          f"{max(e_S):.2e}, rms {max(e_R):.2e}; history {max(e_h):.2e}")
    assert e_x <= TOL_OUT
    assert e_S[0] <= TOL_STATE
    assert max(e_S) <= DRIFT_STATE_MAX, e_S
    assert max(e_R) <= DRIFT_STATE_RMS, e_R
    assert max(e_h) <= TOL_OUT, e_h


def _oracle_inputs(x_in):
    """The oracle's layer input rows as the GPU takes them: the FP32 residual
    (float64 rounded once) and the projection input round_bf16(x) as bf16 bits
    (exactly the value the oracle multiplies)."""
    xb = LY.round_bf16(x_in).astype(np.float32)  # exact: bf16 values are float32 values
    return f32(x_in), bf(W.f32_to_bf16_bits(xb))


def _elem_rel_err(gpu, ref, floor=1e-6):
    """Largest elementwise |gpu - ref| / max(|ref|, floor * max|ref|)."""
    ref = np.asarray(ref, np.float64)
    den = np.maximum(np.abs(ref), floor * np.abs(ref).max())
    return float((np.abs(np.asarray(gpu, np.float64) - ref) / den).max())


def _bf16_decisions(gpu_bits, exact, window=2.0 ** -14, window_row=2.0 ** -18):
    """Check the GPU's bf16 rounding decisions against the exact values
    ([..][d] rows).  Both sides round independently: the oracle its exact
    value, the GPU an FP32 value within tol = window * |x| + window_row *
    max|row| of it (a few units in the last place of the row's projections).
    So each GPU value must be the bf16 rounding of some value within tol of
    the exact one: |g - x| <= half a bf16 unit of g (<= 2^-8 |g|) + tol.
    Returns how many GPU values differ from the oracle's own rounding."""
    x = np.asarray(exact, np.float64)
    r = LY.round_bf16(x)
    g = wide(gpu_bits)
    tol = window * np.abs(x) + window_row * np.abs(x).max(axis=-1, keepdims=True)
    other = g != r
    if other.any():
        xo, go = x[other], g[other]
        bad = np.abs(go - xo) > 2.0 ** -8 * np.abs(go) + tol[other]
        assert not bad.any(), (f"{bad.sum()} bf16 values are not a rounding of a value within "
                               f"the FP32 error of the exact one; worst |gpu - exact| = "
                               f"{np.abs(go - xo)[bad].max():.3e}")
    return int(other.sum())


@pytest.mark.timeout(300)  # 24 layers of weights drawn on the host, three oracle steps
def test_stack_layerwise_matches_oracle_24_layers_three_delayed_steps():
    """Config-5 parity layer by layer and over consecutive steps.  The 24-layer
    stack (hidden 2048, h=8, d=256) runs three speculative steps on 32-node
    window trees with the delayed commit (each step commits the previous
    step's accepted path inside its verification; a flush commits the last).
    Data flows from the oracle to the GPU only:
    - every GPU layer gets the oracle's input rows of that layer and step;
    - its prep (projection, path convolution, SiLU, norms, gates) is checked
      against the oracle's exact values: beta and g to 2e-5, and every bf16
      q, k, v value is the oracle's rounding or, within 2^-14 of a rounding
      midpoint, the other valid rounding (both sides decide independently);
    - its verification and commit then run on the oracle's rounded q, k, v,
      beta, g, so one such decision cannot move a state by a bf16 unit of a
      key: each layer's output is held to 2e-3 and, after every commit, each
      layer's committed state to 1e-3 (max |err| / max |ref| per head), the
      convolution histories (from the GPU's own projections) to 1e-4."""
    shape = W.StackShape(layers=24)
    N, steps = 32, 3
    H, dk, dv = shape.H, shape.dk, shape.dv
    rng, layers, S0 = _stack_case(shape, 1, N, seed=31)
    parents, last = W.stack_drafts(rng, steps, N=N)
    x0 = [W.stack_inputs(rng, N, shape.D) for _ in range(steps)]
    st = _load(shape, layers, S0, 1, N)

    wt = LY.StackWeights([wide(w) for w, _, _ in layers], [c for _, c, _ in layers],
                         [wide(w) for _, _, w in layers], H, dk, dv, bf16=True)
    states = [S0[l][0].astype(np.float64) for l in range(shape.layers)]
    hists = [np.zeros((3, shape.n_conv)) for _ in range(shape.layers)]
    par_t = [i32(parents[s][None]) for s in range(steps)]
    last_t = [i32(last[s:s + 1]) for s in range(steps)]
    worst = dict(out=0.0, state=0.0, hist=0.0, out_elem=0.0, gates=0.0)
    flips = 0

    def check_committed(tag):
        S_gpu = st.S.cpu().numpy()
        h_gpu = st.hist.cpu().numpy()
        for l in range(shape.layers):
            e_S = slice_rel_err(S_gpu[l], states[l][None])
            e_h = rel(h_gpu[l, 0], hists[l])
            worst["state"] = max(worst["state"], e_S)
            worst["hist"] = max(worst["hist"], e_h)
            assert e_S <= TOL_STATE, (tag, l, e_S)
            assert e_h <= 1e-4, (tag, l, e_h)

    for s_ in range(steps):
        x_ref, per_layer = LY.stack_spec_step(wt, wide(x0[s_]), parents[s_], states, hists)
        inputs = [_oracle_inputs(per_layer[l]["x_in"]) for l in range(shape.layers)]
        exact, vin = [], []
        for l in range(shape.layers):
            qx, kx, vx, bx, gx, _ = LY.layer_prep(per_layer[l]["P"], parents[s_], wt.conv_w[l],
                                                  hists[l], H, dk, dv, wt.gate_shift)
            exact.append((qx, kx, vx, bx, gx))
            rb = [W.f32_to_bf16_bits(LY.round_bf16(a).astype(np.float32)[None])
                  for a in (qx, kx, vx)]
            vin.append((bf(rb[0]), bf(rb[1]), bf(rb[2]), f32(bx[None]), f32(gx[None])))
        outs, preps = [], []
        taps = dict(layer_inputs=inputs, layer_outputs=outs, prep_outputs=preps,
                    verify_inputs=vin)
        if s_ == 0:
            st.verify(par_t[0], **taps)
        else:
            st.step(par_t[s_], last_prev=last_t[s_ - 1], parents_prev=par_t[s_ - 1], **taps)
        torch.cuda.synchronize()
        st.check_status()
        if s_ > 0:  # the previous step's path is now committed on the GPU
            check_committed(f"after step {s_ - 1}")
        for l in range(shape.layers):
            qx, kx, vx, bx, gx = exact[l]
            gq, gk, gv, gb, gg = preps[l]
            for got, ex in ((gq, qx), (gk, kx), (gv, vx)):
                flips += _bf16_decisions(bits_of(got)[0], ex)
            for got, ex in ((gb, bx), (gg, gx)):
                e = np.abs(got.cpu().numpy()[0] - ex) / np.maximum(np.abs(ex), 1e-6)
                worst["gates"] = max(worst["gates"], float(e.max()))
            assert worst["gates"] <= 2e-5, (s_, l, worst["gates"])
            ref = per_layer[l + 1]["x_in"] if l + 1 < shape.layers else x_ref
            got = outs[l].cpu().numpy()
            e = rel(got, ref)
            worst["out"] = max(worst["out"], e)
            worst["out_elem"] = max(worst["out_elem"], _elem_rel_err(got, ref))
            assert e <= TOL_OUT, (s_, l, e)
        states, hists = LY.stack_commit(wt, parents[s_], states, hists, per_layer, int(last[s_]))
    st.flush(par_t[-1], last_t[-1])
    torch.cuda.synchronize()
    st.check_status()
    check_committed(f"after step {steps - 1}")
    total = steps * shape.layers * N * H * (2 * dk + dv)
    print(f"\n24 layers x {steps} delayed steps, oracle-fed: outputs {worst['out']:.2e} "
          f"(elementwise, floor 1e-6: {worst['out_elem']:.2e}); committed states "
          f"{worst['state']:.2e}; histories {worst['hist']:.2e}; beta, g {worst['gates']:.2e}; "
          f"bf16 q/k/v decisions at a midpoint taken the other way: {flips} of {total}")


def test_stack_chain_verify_equals_token_by_token_decode():
    """The stack's layer-major verification of an 8-node chain, then the
    commit of all 8 nodes, gives the same outputs, states and histories as
    8 one-token decode steps (both on the GPU)."""
    shape = W.StackShape(layers=3, D=512, H=8, dk=64, dv=64)
    N = 8
    rng, layers, S0 = _stack_case(shape, 1, N, seed=4)
    x0 = W.stack_inputs(rng, N, shape.D)
    spec = _load(shape, layers, S0, 1, N)
    spec.set_inputs(f32(wide(x0)), bf(x0))
    par = i32(W.chain_parents(N)[None])
    spec.verify(par)
    spec.commit(par, i32([N - 1]))
    ar = _load(shape, layers, S0, 1, N)
    outs = []
    for t in range(N):
        ar.ar_step(f32(wide(x0[t:t + 1])), bf(x0[t:t + 1]))
        outs.append(ar.x1.clone())
    torch.cuda.synchronize()
    x_ar = torch.cat(outs).cpu().numpy().astype(np.float64)
    e_x = rel(spec.x.cpu().numpy(), x_ar)
    S_ar = ar.S.cpu().numpy().astype(np.float64)
    S_sp = spec.S.cpu().numpy()
    e_S = [slice_rel_err(S_sp[l], S_ar[l]) for l in range(shape.layers)]
    e_R = [rms_rel_err(S_sp[l, 0], S_ar[l, 0]) for l in range(shape.layers)]
    e_h = [rel(spec.hist[l].cpu().numpy(), ar.hist[l].cpu().numpy().astype(np.float64))
           for l in range(shape.layers)]
    print(f"\nchain vs token-by-token: output {e_x:.2e}; layer-0 state {e_S[0]:.2e}; "
          f"states max {max(e_S):.2e}, rms {max(e_R):.2e}; history {max(e_h):.2e}")
    assert e_x <= TOL_OUT
    assert e_S[0] <= TOL_STATE
    assert max(e_S) <= DRIFT_STATE_MAX and max(e_R) <= DRIFT_STATE_RMS
    assert max(e_h) <= TOL_OUT
    # layer 0 sees identical inputs on both routes: its projection rows match bitwise
    assert torch.equal(spec.hist[0], ar.hist[0])


def test_stack_delayed_commit_is_bitwise_the_two_step_path():
    """Two speculative steps with the delayed commit (then a flush) leave the
    stack bitwise where verify / commit / verify / commit leaves it."""
    shape = W.StackShape(layers=3, D=512, H=8, dk=64, dv=64)
    N = 16
    rng, layers, S0 = _stack_case(shape, 1, N, seed=8)
    parents, last = W.stack_drafts(rng, 2, N=N)
    x0 = [W.stack_inputs(rng, N, shape.D) for _ in range(2)]
    par = [i32(parents[s][None]) for s in range(2)]
    lst = [i32(last[s:s + 1]) for s in range(2)]
    a = _load(shape, layers, S0, 1, N)
    b = _load(shape, layers, S0, 1, N)
    outs_a, outs_b = [], []
    for s_ in range(2):
        a.set_inputs(f32(wide(x0[s_])), bf(x0[s_]))
        a.verify(par[s_])
        a.commit(par[s_], lst[s_])
        outs_a.append(a.x.clone())
        b.set_inputs(f32(wide(x0[s_])), bf(x0[s_]))
        if s_ == 0:
            b.verify(par[0])
        else:
            b.step(par[1], last_prev=lst[0], parents_prev=par[0])
        outs_b.append(b.x.clone())
    b.flush(par[1], lst[1])
    torch.cuda.synchronize()
    for xa, xb_ in zip(outs_a, outs_b):
        assert torch.equal(xa, xb_)
    assert torch.equal(a.S, b.S)
    assert torch.equal(a.hist, b.hist)
