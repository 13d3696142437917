"""Host-side checks of libgdnspec: it loads, exports what gdnspec.h declares,
computes layouts, and rejects bad arguments before touching the GPU."""

import ctypes

import pytest

from linear_attention_gdn_amd import gdnspec as G


def test_library_exports_every_declared_function():
    names = G.declared_functions()
    assert {"gdn_tree_verify", "gdn_chain_verify", "gdn_commit_path", "gdn_factor_bytes",
            "gdn_factor_layout", "gdn_workspace_bytes", "gdn_last_error",
            "gdn_version"} <= set(names)
    L = G.lib()
    for n in names:
        assert hasattr(L, n), n
    assert G.gdn_version() >= 1


def test_factor_layout_sections():
    B, N, H, dk, dv = 8, 64, 8, 256, 256
    for code, esize in ((G.GDN_BF16, 2), (G.GDN_F32, 4)):
        off = G.gdn_factor_layout(B, N, H, dk, dv, code)
        sizes = [B * H * N * dv * 4, B * H * N * 4, B * H * N * dk * esize, B * N * 4, B * N * 8]
        assert off[0] == 0
        for i in range(5):
            assert off[i] % 256 == 0
            end = off[i] + sizes[i]
            nxt = off[i + 1] if i < 4 else G.gdn_factor_bytes(B, N, H, dk, dv, code)
            assert end <= nxt < end + 256
    assert G.gdn_workspace_bytes(B, N, H, dk, dv) == 0  # no scratch in this version


@pytest.mark.parametrize("sizes", [(1, 65, 8, 256, 256), (1, 8, 8, 12, 256), (1, 8, 8, 256, 6),
                                   (1, 8, 0, 256, 256), (-1, 8, 8, 256, 256),
                                   (1, 8, 8, 264, 256), (1, 8, 8, 256, 260)])
def test_bad_sizes_rejected(sizes):
    assert G.gdn_factor_bytes(*sizes, G.GDN_BF16) == 0
    P = ctypes.c_void_p(4096)
    rc = G.lib().gdn_tree_verify(*sizes, G.GDN_BF16, P, P, P, P, P, P, P, 1.0, P, P, P, None,
                                 None, None)
    assert rc == G.GDN_ERR_SHAPE
    assert "unsupported sizes" in G.gdn_last_error()
    rc = G.lib().gdn_chain_verify(*sizes, G.GDN_BF16, P, P, P, P, P, P, 1.0, P, P, None)
    assert rc == G.GDN_ERR_SHAPE
    rc = G.lib().gdn_commit_path(*sizes, G.GDN_BF16, P, P, P, None, None, None, None)
    assert rc == G.GDN_ERR_SHAPE


def test_bad_pointers_and_dtype_rejected():
    L = G.lib()
    P = ctypes.c_void_p(4096)
    odd = ctypes.c_void_p(4096 + 8)
    sz = (1, 8, 8, 256, 256)
    assert L.gdn_tree_verify(*sz, 7, P, P, P, P, P, P, P, 1.0, P, P, P, None, None,
                             None) == G.GDN_ERR_ARG
    assert "qkv_dtype" in G.gdn_last_error()
    assert L.gdn_tree_verify(*sz, 0, None, P, P, P, P, P, P, 1.0, P, P, P, None, None,
                             None) == G.GDN_ERR_ARG
    assert "S0 is NULL" in G.gdn_last_error()
    assert L.gdn_tree_verify(*sz, 0, odd, P, P, P, P, P, P, 1.0, P, P, P, None, None,
                             None) == G.GDN_ERR_ARG
    assert "aligned" in G.gdn_last_error()
    assert L.gdn_tree_verify(*sz, 0, P, P, P, P, P, P, P, float("nan"), P, P, P, None, None,
                             None) == G.GDN_ERR_ARG
    assert L.gdn_chain_verify(*sz, 0, P, P, P, P, P, P, 1.0, P, None, None) == G.GDN_ERR_ARG
    assert "factors is NULL" in G.gdn_last_error()
    assert L.gdn_commit_path(*sz, 0, P, P, None, None, None, None, None) == G.GDN_ERR_ARG
    assert "last_accepted is NULL" in G.gdn_last_error()


def test_chain_lds_limit_rejected():
    """The chain kernel stages the draft (and, delayed, the previous record) in
    one workgroup's LDS; fp32 inputs at the largest sizes exceed 160 KiB and
    are refused before any launch, bf16 at the same sizes fits."""
    L = G.lib()
    P = ctypes.c_void_p(4096)
    P2 = ctypes.c_void_p(1 << 30)
    sz = (1, 64, 64, 8, 256, 256)  # B, N_prev, N, H, dk, dv
    rc = L.gdn_chain_verify_delayed(*sz, G.GDN_F32, P, P2, P, None, P, P, P, P, P, 1.0, P, P,
                                    None)
    assert rc == G.GDN_ERR_UNSUPPORTED
    assert "LDS" in G.gdn_last_error()


def test_empty_problems_are_noops():
    L = G.lib()
    assert L.gdn_tree_verify(0, 8, 8, 256, 256, 0, None, None, None, None, None, None, None,
                             1.0, None, None, None, None, None, None) == G.GDN_OK
    assert L.gdn_chain_verify(1, 0, 8, 256, 256, 0, None, None, None, None, None, None, 1.0,
                              None, None, None) == G.GDN_OK
    assert L.gdn_commit_path(0, 8, 8, 256, 256, 0, None, None, None, None, None, None,
                             None) == G.GDN_OK
    assert G.gdn_last_error() == ""


def test_binding_refuses_host_tensors():
    import torch
    S0 = torch.zeros(1, 1, 16, 16)
    q = torch.zeros(1, 4, 1, 16)
    with pytest.raises(ValueError):
        G.gdn_chain_verify(S0, q, q, q, torch.zeros(1, 4, 1), torch.zeros(1, 4, 1),
                           torch.zeros(1, 4, 1, 16), None)


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(G, "_lib", None)
    monkeypatch.setattr(G, "LIB_PATH", "/nonexistent/libgdnspec.so")
    with pytest.raises(RuntimeError, match="missing"):
        G.lib()


def test_layer_scaffold_exports():
    assert {"gdn_linear", "gdn_pack_weights", "gdn_layer_prep", "gdn_gate_merge",
            "gdn_conv_commit", "gdn_decode_step", "gdn_layer_verify",
            "gdn_layer_prep_delayed"} <= set(G.declared_functions())


@pytest.mark.parametrize("mnk", [(65, 16, 512), (4, 24, 512), (4, 16, 384), (4, 16, 128),
                                 (-1, 16, 512), (4, 16, 131072)])
def test_linear_bad_sizes_rejected(mnk):
    P = ctypes.c_void_p(4096)
    assert G.lib().gdn_linear(*mnk, P, P, 0, None, P, None, None) == G.GDN_ERR_SHAPE
    assert "unsupported sizes" in G.gdn_last_error()


def test_layer_scaffold_bad_arguments_rejected():
    L = G.lib()
    P = ctypes.c_void_p(4096)
    odd = ctypes.c_void_p(4096 + 4)
    assert L.gdn_linear(4, 16, 512, P, P, 0, None, None, None, None) == G.GDN_ERR_ARG
    assert "both NULL" in G.gdn_last_error()
    assert L.gdn_linear(4, 16, 512, None, P, 0, None, P, None, None) == G.GDN_ERR_ARG
    assert L.gdn_linear(4, 16, 512, P, odd, 0, None, P, None, None) == G.GDN_ERR_ARG
    assert L.gdn_linear(4, 16, 512, P, P, 2, None, P, None, None) == G.GDN_ERR_ARG
    assert "w_layout" in G.gdn_last_error()
    assert L.gdn_linear(0, 16, 512, None, None, 1, None, P, None, None) == G.GDN_OK
    assert L.gdn_pack_weights(24, 512, P, P, None) == G.GDN_ERR_SHAPE
    assert L.gdn_pack_weights(16, 512, P, ctypes.c_void_p(4096 + 1024), None) == G.GDN_ERR_ARG
    assert "overlap" in G.gdn_last_error()
    # prep: sizes follow the verifier's limits; D % 8 == 0; gate_shift must be finite
    assert L.gdn_layer_prep(1, 65, 8, 256, 256, 2048, P, P, P, P, P, P, 2.0, P, P, P, P, P,
                            None) == G.GDN_ERR_SHAPE
    assert L.gdn_layer_prep(1, 8, 8, 256, 256, 2044, P, P, P, P, P, P, 2.0, P, P, P, P, P,
                            None) == G.GDN_ERR_SHAPE
    assert "hidden width" in G.gdn_last_error()
    assert L.gdn_layer_prep(1, 8, 8, 256, 256, 2048, P, P, P, P, P, P, float("inf"), P, P, P,
                            P, P, None) == G.GDN_ERR_ARG
    assert L.gdn_layer_prep(1, 8, 8, 256, 256, 2048, P, P, P, P, None, P, 2.0, P, P, P, P, P,
                            None) == G.GDN_ERR_ARG
    assert "conv_w is NULL" in G.gdn_last_error()
    assert L.gdn_layer_prep(1, 8, 8, 256, 256, 2048, P, P, None, P, P, P, 2.0, P, P, P, P, P,
                            None) == G.GDN_ERR_ARG
    assert "W_ab is NULL" in G.gdn_last_error()
    assert L.gdn_layer_prep(0, 8, 8, 256, 256, 2048, None, None, None, None, None, None, 2.0,
                            None, None, None, None, None, None) == G.GDN_OK
    # gate merge
    assert L.gdn_gate_merge(4, 6, P, P, 8, P, None) == G.GDN_ERR_SHAPE
    assert L.gdn_gate_merge(4, 8, P, P, 4, P, None) == G.GDN_ERR_SHAPE
    assert L.gdn_gate_merge(4, 8, P, P, 8, None, None) == G.GDN_ERR_ARG
    assert L.gdn_gate_merge(0, 8, None, None, 8, None, None) == G.GDN_OK
    # conv commit
    assert L.gdn_conv_commit(1, 65, 16, P, 16, P, P, P, None, None) == G.GDN_ERR_SHAPE
    assert L.gdn_conv_commit(1, 8, 18, P, 20, P, P, P, None, None) == G.GDN_ERR_SHAPE
    assert L.gdn_conv_commit(1, 8, 16, P, 12, P, P, P, None, None) == G.GDN_ERR_SHAPE
    assert L.gdn_conv_commit(1, 8, 16, P, 16, P, None, P, None, None) == G.GDN_ERR_ARG
    assert L.gdn_conv_commit(0, 8, 16, None, 16, None, None, None, None, None) == G.GDN_OK
    # decode step
    assert L.gdn_decode_step(1, 8, 12, 256, 0, P, P, P, P, P, P, 1.0, P,
                             None) == G.GDN_ERR_SHAPE
    assert L.gdn_decode_step(1, 8, 256, 256, 5, P, P, P, P, P, P, 1.0, P,
                             None) == G.GDN_ERR_ARG
    assert L.gdn_decode_step(1, 8, 256, 256, 0, P, P, P, P, P, P, 1.0, None,
                             None) == G.GDN_ERR_ARG
    assert "out is NULL" in G.gdn_last_error()
    assert L.gdn_decode_step(0, 8, 256, 256, 0, None, None, None, None, None, None, 1.0, None,
                             None) == G.GDN_OK
    # gated layer verify: gate row length, gate and Y required, N_prev when delayed
    lv = lambda B, Np, N, prev, gate, ldg, Y: L.gdn_layer_verify(
        B, Np, N, 8, 256, 256, P, prev, P, None, P, P, P, P, P, P, 1.0, gate, ldg, Y, P, None,
        None)
    assert lv(1, 32, 32, P, P, 2047, P) == G.GDN_ERR_SHAPE
    assert "ldg" in G.gdn_last_error()
    assert lv(1, 32, 32, P, P, 2048, None) == G.GDN_ERR_ARG
    assert "Y is NULL" in G.gdn_last_error()
    assert lv(1, 32, 32, P, None, 2048, P) == G.GDN_ERR_ARG
    assert lv(1, 0, 32, P, P, 2048, P) == G.GDN_ERR_SHAPE
    assert "N_prev" in G.gdn_last_error()
    assert lv(1, 65, 32, P, P, 2048, P) == G.GDN_ERR_SHAPE
    assert lv(1, 0, 65, None, P, 2048, P) == G.GDN_ERR_SHAPE
    assert lv(0, 0, 32, None, None, 2048, None) == G.GDN_OK
    # fused history commit + prep: N_prev range, previous-step pointers, distinct histories
    pd = lambda Np, N, hist, P_prev, hist_out: L.gdn_layer_prep_delayed(
        1, Np, N, 8, 256, 256, 2048, P, P, P, P, P, hist, 2.0, P, P, P, P, P, P_prev, P, P,
        hist_out, None, None)
    H2 = ctypes.c_void_p(4096 + (1 << 20))
    assert pd(0, 32, P, P, H2) == G.GDN_ERR_SHAPE
    assert pd(65, 32, P, P, H2) == G.GDN_ERR_SHAPE
    assert pd(32, 32, P, None, H2) == G.GDN_ERR_ARG
    assert "P_prev is NULL" in G.gdn_last_error()
    assert pd(32, 32, P, P, P) == G.GDN_ERR_ARG
    assert "overlap" in G.gdn_last_error()
    assert pd(32, 0, P, P, H2) == G.GDN_ERR_SHAPE


def test_layer_bindings_refuse_host_tensors():
    import torch
    A = torch.zeros(4, 512, dtype=torch.bfloat16)
    W = torch.zeros(16, 512, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        G.gdn_linear(A, W, C=torch.zeros(4, 16))


def test_replay_entry_points_validate_arguments():
    L = G.lib()
    P = ctypes.c_void_p(4096)
    sz = (1, 8, 8, 256, 256)
    for bad_p in (0, 65):
        assert L.gdn_replay_verify(*sz, 0, P, P, P, P, P, P, P, 1.0, P, bad_p, P, None,
                                   None) == G.GDN_ERR_SHAPE
        assert "path slots" in G.gdn_last_error()
    assert L.gdn_replay_verify(*sz, 0, P, P, P, P, P, P, P, 1.0, None, 4, P, None,
                               None) == G.GDN_ERR_ARG
    assert "ends is NULL" in G.gdn_last_error()
    assert L.gdn_replay_verify(1, 65, 8, 256, 256, 0, P, P, P, P, P, P, P, 1.0, P, 4, P, None,
                               None) == G.GDN_ERR_SHAPE
    assert L.gdn_replay_commit(*sz, 0, P, P, P, P, P, P, None, None, None) == G.GDN_ERR_ARG
    assert "last_accepted is NULL" in G.gdn_last_error()
    assert L.gdn_replay_commit(*sz, 5, P, P, P, P, P, P, P, None, None) == G.GDN_ERR_ARG


def test_prune_entry_point_validates_arguments():
    L = G.lib()
    P = ctypes.c_void_p(4096)
    for B, M, T in ((1, 0, 4), (1, 1025, 4), (1, 10, 0), (1, 10, 65), (-1, 10, 4)):
        assert L.gdn_prune_draft(B, M, T, 1.0, P, P, P, P, P, None, None) == G.GDN_ERR_SHAPE
    for tau in (float("nan"), float("inf"), -0.5):
        assert L.gdn_prune_draft(1, 10, 4, tau, P, P, P, P, P, None, None) == G.GDN_ERR_ARG
    assert L.gdn_prune_draft(1, 10, 4, 1.0, P, None, P, P, P, None, None) == G.GDN_ERR_ARG
    assert "conf is NULL" in G.gdn_last_error()
