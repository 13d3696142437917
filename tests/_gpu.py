"""Helpers for the GPU parity tests: move seeded drafts to the device, run the
library through its C ABI, and measure errors against the oracle."""

from __future__ import annotations

import numpy as np
import torch

from linear_attention_gdn_amd import gdnspec as G
from linear_attention_gdn_amd import workloads as W

# Tolerances: max |gpu - oracle| / max |oracle| per (sequence, head) slice.
TOL_OUT = 2e-3    # outputs
TOL_UP = 2e-3     # factor-record state writes u'
TOL_STATE = 1e-3  # committed state


def dev_tensors(d: W.Draft, device="cuda"):
    def qkv(x):
        if d.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16).copy()).to(
                device).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device)

    f = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device)
    i = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(device)
    return dict(S0=f(d.S0), q=qkv(d.q), k=qkv(d.k), v=qkv(d.v), beta=f(d.beta), g=f(d.g),
                parents=i(d.parents), last=i(d.last_accepted))


def code_of(d: W.Draft) -> int:
    return G.GDN_BF16 if d.dtype == "bf16" else G.GDN_F32


def run_tree(d: W.Draft, t=None):
    t = t or dev_tensors(d)
    B, N, H, dk, dv = d.B, d.N, d.H, d.dk, d.dv
    out = torch.full((B, N, H, dv), float("nan"), device="cuda")
    rec = G.FactorRecord.empty(B, N, H, dk, dv, code_of(d))
    mask = torch.zeros((B, N), dtype=torch.int64, device="cuda")
    st = torch.full((B,), 77, dtype=torch.int32, device="cuda")
    G.gdn_tree_verify(t["S0"], t["parents"], t["q"], t["k"], t["v"], t["beta"], t["g"], out,
                      rec, None, scale=d.scale, mask_out=mask, dev_status=st)
    torch.cuda.synchronize()
    return out, rec, mask, st, t


def run_chain(d: W.Draft, t=None):
    t = t or dev_tensors(d)
    B, N, H, dk, dv = d.B, d.N, d.H, d.dk, d.dv
    out = torch.full((B, N, H, dv), float("nan"), device="cuda")
    rec = G.FactorRecord.empty(B, N, H, dk, dv, code_of(d))
    G.gdn_chain_verify(t["S0"], t["q"], t["k"], t["v"], t["beta"], t["g"], out, rec,
                       scale=d.scale)
    torch.cuda.synchronize()
    return out, rec, t


def run_commit(d: W.Draft, rec: G.FactorRecord, S0: torch.Tensor, last):
    S = S0.clone()
    last_t = torch.as_tensor(np.asarray(last, np.int32)).cuda()
    path = torch.full((d.B, d.N), 99, dtype=torch.int32, device="cuda")
    plen = torch.full((d.B,), 99, dtype=torch.int32, device="cuda")
    st = torch.full((d.B,), 77, dtype=torch.int32, device="cuda")
    G.gdn_commit_path(S, rec, last_t, path_out=path, path_len_out=plen, dev_status=st)
    torch.cuda.synchronize()
    return S, path, plen, st


def slice_rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """Largest per-(b, h) ratio max|gpu - ref| / max|ref|; inputs shaped [B][H][...]."""
    B, H = ref.shape[:2]
    worst = 0.0
    for b in range(B):
        for h in range(H):
            r = ref[b, h]
            den = np.abs(r).max()
            num = np.abs(gpu[b, h].astype(np.float64) - r).max()
            if den == 0.0:
                if num != 0.0:
                    return float("inf")
                continue
            worst = max(worst, num / den)
    return worst


def elem_rel_err(gpu: np.ndarray, ref: np.ndarray, floor: float = 1e-6) -> float:
    """Largest elementwise |gpu - ref| / max(|ref|, floor * max|ref| of the slice)
    per (b, h) slice; inputs shaped [B][H][...].  Reported beside
    slice_rel_err (the gated metric): it shows how small elements fare."""
    B, H = ref.shape[:2]
    worst = 0.0
    for b in range(B):
        for h in range(H):
            r = np.asarray(ref[b, h], np.float64)
            den = np.maximum(np.abs(r), floor * np.abs(r).max())
            if not den.any():
                continue
            worst = max(worst, float((np.abs(gpu[b, h].astype(np.float64) - r) / den).max()))
    return worst


def out_err(out_gpu: torch.Tensor, out_ref: np.ndarray) -> float:
    """Outputs are [B][N][H][dv]; compare per (b, h)."""
    g = out_gpu.cpu().numpy().transpose(0, 2, 1, 3)
    return slice_rel_err(g, out_ref.transpose(0, 2, 1, 3))


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()
