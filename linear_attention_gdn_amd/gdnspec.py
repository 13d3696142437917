"""ctypes binding of libgdnspec (``include/gdnspec.h``, ``include/gdnlayer.h``,
``include/gdnnext.h``),
with the same names.

Argument marshalling only: every step of verification, commit and the layer
scaffold runs in the HIP kernels of ``libgdnspec.so``.  PyTorch supplies device memory and the
current HIP stream.  There is no fallback: if the library is missing the
calls raise.
"""

from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdnspec.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
HEADERS = [os.path.join(INCLUDE, "gdnspec.h"), os.path.join(INCLUDE, "gdnlayer.h"),
           os.path.join(INCLUDE, "gdnnext.h")]

GDN_OK = 0
GDN_ERR_ARG = -1
GDN_ERR_SHAPE = -2
GDN_ERR_TOPOLOGY = -3
GDN_ERR_UNSUPPORTED = -4
GDN_ERR_HIP = -5
GDN_BF16 = 0
GDN_F32 = 1
GDN_W_ROWS = 0
GDN_W_PACKED = 1

_lib = None


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libgdnspec.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m linear_attention_gdn_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        I, P, F, S = ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
        L.gdn_version.argtypes = []
        L.gdn_version.restype = I
        L.gdn_last_error.argtypes = []
        L.gdn_last_error.restype = ctypes.c_char_p
        L.gdn_factor_bytes.argtypes = [I, I, I, I, I, I]
        L.gdn_factor_bytes.restype = S
        L.gdn_factor_layout.argtypes = [I, I, I, I, I, I, ctypes.POINTER(S)]
        L.gdn_factor_layout.restype = I
        L.gdn_workspace_bytes.argtypes = [I, I, I, I, I]
        L.gdn_workspace_bytes.restype = S
        L.gdn_tree_verify.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, F, P, P, P, P, P, P]
        L.gdn_tree_verify.restype = I
        L.gdn_chain_verify.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, F, P, P, P]
        L.gdn_chain_verify.restype = I
        L.gdn_commit_path.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P]
        L.gdn_commit_path.restype = I
        L.gdn_chain_verify_delayed.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, F,
                                               P, P, P]
        L.gdn_chain_verify_delayed.restype = I
        L.gdn_tree_verify_delayed.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P,
                                              F, P, P, P, P, P, P]
        L.gdn_tree_verify_delayed.restype = I
        L.gdn_linear.argtypes = [I, I, I, P, P, I, P, P, P, P]
        L.gdn_linear.restype = I
        L.gdn_pack_weights.argtypes = [I, I, P, P, P]
        L.gdn_pack_weights.restype = I
        L.gdn_layer_prep.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, F, P, P, P, P, P, P]
        L.gdn_layer_prep.restype = I
        L.gdn_gate_merge.argtypes = [I, I, P, P, I, P, P]
        L.gdn_gate_merge.restype = I
        L.gdn_layer_verify.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, F, P, I,
                                       P, P, P, P]
        L.gdn_layer_verify.restype = I
        L.gdn_layer_prep_delayed.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, F, P, P, P,
                                             P, P, P, P, P, P, P, P]
        L.gdn_layer_prep_delayed.restype = I
        L.gdn_conv_commit.argtypes = [I, I, I, P, I, P, P, P, P, P]
        L.gdn_conv_commit.restype = I
        L.gdn_decode_step.argtypes = [I, I, I, I, I, P, P, P, P, P, P, F, P, P]
        L.gdn_decode_step.restype = I
        L.gdn_replay_verify.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, F, P, I, P, P, P]
        L.gdn_replay_verify.restype = I
        L.gdn_replay_commit.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P]
        L.gdn_replay_commit.restype = I
        L.gdn_hybrid_plan_entries.argtypes = [I, I]
        L.gdn_hybrid_plan_entries.restype = S
        L.gdn_hybrid_plan.argtypes = [I, I, P, P, P, P]
        L.gdn_hybrid_plan.restype = I
        L.gdn_hybrid_verify.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, F, P, P, P, I, P,
                                        P, P]
        L.gdn_hybrid_verify.restype = I
        L.gdn_prune_draft.argtypes = [I, I, I, F, P, P, P, P, P, P, P]
        L.gdn_prune_draft.restype = I
        _lib = L
    return _lib


def declared_functions() -> list:
    """Names of the functions the headers under ``include/`` declare."""
    names = set()
    for path in HEADERS:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text))
    return sorted(names)


def gdn_version() -> int:
    return int(lib().gdn_version())


def gdn_last_error() -> str:
    return lib().gdn_last_error().decode()


def _raise_on(status: int):
    if status != GDN_OK:
        raise GdnError(status, gdn_last_error())


def dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return GDN_BF16
    if t == torch.float32:
        return GDN_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t}")


def torch_dtype(code: int) -> torch.dtype:
    return torch.bfloat16 if code == GDN_BF16 else torch.float32


def gdn_factor_bytes(B, N, H, dk, dv, qkv_dtype) -> int:
    return int(lib().gdn_factor_bytes(B, N, H, dk, dv, qkv_dtype))


def gdn_factor_layout(B, N, H, dk, dv, qkv_dtype) -> tuple:
    off = (ctypes.c_size_t * 5)()
    _raise_on(lib().gdn_factor_layout(B, N, H, dk, dv, qkv_dtype, off))
    return tuple(int(x) for x in off)


def gdn_workspace_bytes(B, N, H, dk, dv) -> int:
    return int(lib().gdn_workspace_bytes(B, N, H, dk, dv))


@dataclass
class FactorRecord:
    """Device buffer holding one verification's factor record, plus its sizes."""

    buf: torch.Tensor  # uint8, gdn_factor_bytes(...)
    B: int
    N: int
    H: int
    dk: int
    dv: int
    qkv_dtype: int

    @classmethod
    def empty(cls, B, N, H, dk, dv, qkv_dtype, device="cuda") -> "FactorRecord":
        n = gdn_factor_bytes(B, N, H, dk, dv, qkv_dtype)
        if n == 0:
            raise GdnError(GDN_ERR_SHAPE, f"unsupported sizes B={B} N={N} H={H} dk={dk} dv={dv}")
        return cls(torch.empty(n, dtype=torch.uint8, device=device), B, N, H, dk, dv, qkv_dtype)

    def _section(self, i, dtype, shape):
        off = gdn_factor_layout(self.B, self.N, self.H, self.dk, self.dv, self.qkv_dtype)[i]
        count = 1
        for s in shape:
            count *= s
        nbytes = count * torch.empty((), dtype=dtype).element_size()
        return self.buf[off:off + nbytes].view(dtype).view(shape)

    @property
    def uprime(self):
        return self._section(0, torch.float32, (self.B, self.H, self.N, self.dv))

    @property
    def G(self):
        return self._section(1, torch.float32, (self.B, self.H, self.N))

    @property
    def K(self):
        return self._section(2, torch_dtype(self.qkv_dtype), (self.B, self.H, self.N, self.dk))

    @property
    def parents(self):
        return self._section(3, torch.int32, (self.B, self.N))

    @property
    def mask(self):
        return self._section(4, torch.int64, (self.B, self.N))


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(name, t, shape, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_draft(S0, q, k, v, beta, g):
    if S0.dim() != 4:
        raise ValueError("S0 must be [B][H][dv][dk]")
    B, H, dv, dk = S0.shape
    if q.dim() != 4:
        raise ValueError("q must be [B][N][H][dk]")
    N = q.shape[1]
    dt = q.dtype
    _need("S0", S0, (B, H, dv, dk), torch.float32)
    _need("q", q, (B, N, H, dk), dt)
    _need("k", k, (B, N, H, dk), dt)
    _need("v", v, (B, N, H, dv), dt)
    _need("beta", beta, (B, N, H), torch.float32)
    _need("g", g, (B, N, H), torch.float32)
    return B, N, H, dk, dv, dtype_code(dt)


def _check_record(rec: FactorRecord, B, N, H, dk, dv, code):
    if (rec.B, rec.N, rec.H, rec.dk, rec.dv, rec.qkv_dtype) != (B, N, H, dk, dv, code):
        raise ValueError("factor record sizes do not match the call")


def gdn_tree_verify(S0, parents, q, k, v, beta, g, out, factors: FactorRecord,
                    workspace: Optional[torch.Tensor] = None, scale: float = 1.0,
                    mask_out=None, dev_status=None, stream=None) -> None:
    """Tree-masked factorized verification; see ``gdn_tree_verify`` in gdnspec.h."""
    B, N, H, dk, dv, code = _check_draft(S0, q, k, v, beta, g)
    _need("parents", parents, (B, N), torch.int32)
    _need("out", out, (B, N, H, dv), torch.float32)
    _check_record(factors, B, N, H, dk, dv, code)
    need = gdn_workspace_bytes(B, N, H, dk, dv)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        raise ValueError("workspace is smaller than gdn_workspace_bytes()")
    if mask_out is not None:
        _need("mask_out", mask_out, (B, N), torch.int64)
    if dev_status is not None:
        _need("dev_status", dev_status, (B,), torch.int32)
    _raise_on(lib().gdn_tree_verify(B, N, H, dk, dv, code, _p(S0), _p(parents), _p(q), _p(k),
                                    _p(v), _p(beta), _p(g), float(scale), _p(out),
                                    _p(factors.buf), _p(workspace), _p(mask_out),
                                    _p(dev_status), _stream(stream)))


def gdn_chain_verify(S0, q, k, v, beta, g, out, factors: FactorRecord, scale: float = 1.0,
                     stream=None) -> None:
    """Serial V-tiled chain verification; see ``gdn_chain_verify`` in gdnspec.h."""
    B, N, H, dk, dv, code = _check_draft(S0, q, k, v, beta, g)
    _need("out", out, (B, N, H, dv), torch.float32)
    _check_record(factors, B, N, H, dk, dv, code)
    _raise_on(lib().gdn_chain_verify(B, N, H, dk, dv, code, _p(S0), _p(q), _p(k), _p(v),
                                     _p(beta), _p(g), float(scale), _p(out), _p(factors.buf),
                                     _stream(stream)))


def gdn_chain_verify_delayed(S, prev_factors: FactorRecord, last_accepted, q, k, v, beta, g,
                             out, factors: FactorRecord, scale: float = 1.0, dev_status=None,
                             stream=None) -> None:
    """Apply the previous record's accepted path to S, then verify a new chain,
    in one pass; see ``gdn_chain_verify_delayed`` in gdnspec.h."""
    B, N, H, dk, dv, code = _check_draft(S, q, k, v, beta, g)
    _need("out", out, (B, N, H, dv), torch.float32)
    _check_record(factors, B, N, H, dk, dv, code)
    pf = prev_factors
    if (pf.B, pf.H, pf.dk, pf.dv, pf.qkv_dtype) != (B, H, dk, dv, code):
        raise ValueError("prev_factors sizes do not match the call")
    _need("last_accepted", last_accepted, (B,), torch.int32)
    if dev_status is not None:
        _need("dev_status", dev_status, (B,), torch.int32)
    _raise_on(lib().gdn_chain_verify_delayed(B, pf.N, N, H, dk, dv, code, _p(S), _p(pf.buf),
                                             _p(last_accepted), _p(dev_status), _p(q), _p(k),
                                             _p(v), _p(beta), _p(g), float(scale), _p(out),
                                             _p(factors.buf), _stream(stream)))


def gdn_tree_verify_delayed(S, prev_factors: FactorRecord, last_accepted, parents, q, k, v,
                            beta, g, out, factors: FactorRecord, workspace=None,
                            scale: float = 1.0, commit_status=None, mask_out=None,
                            dev_status=None, stream=None) -> None:
    """Apply the previous record's accepted path to S, then verify a new tree,
    in one pass; see ``gdn_tree_verify_delayed`` in gdnspec.h."""
    B, N, H, dk, dv, code = _check_draft(S, q, k, v, beta, g)
    _need("parents", parents, (B, N), torch.int32)
    _need("out", out, (B, N, H, dv), torch.float32)
    _check_record(factors, B, N, H, dk, dv, code)
    pf = prev_factors
    if (pf.B, pf.H, pf.dk, pf.dv, pf.qkv_dtype) != (B, H, dk, dv, code):
        raise ValueError("prev_factors sizes do not match the call")
    _need("last_accepted", last_accepted, (B,), torch.int32)
    for name, t in (("commit_status", commit_status), ("dev_status", dev_status)):
        if t is not None:
            _need(name, t, (B,), torch.int32)
    if mask_out is not None:
        _need("mask_out", mask_out, (B, N), torch.int64)
    _raise_on(lib().gdn_tree_verify_delayed(B, pf.N, N, H, dk, dv, code, _p(S), _p(pf.buf),
                                            _p(last_accepted), _p(commit_status), _p(parents),
                                            _p(q), _p(k), _p(v), _p(beta), _p(g), float(scale),
                                            _p(out), _p(factors.buf), _p(workspace),
                                            _p(mask_out), _p(dev_status), _stream(stream)))


def gdn_commit_path(S, factors: FactorRecord, last_accepted, path_out=None, path_len_out=None,
                    dev_status=None, stream=None) -> None:
    """Apply the accepted path's buffered factors to S in place; see gdnspec.h."""
    B, N, H, dk, dv = factors.B, factors.N, factors.H, factors.dk, factors.dv
    _need("S", S, (B, H, dv, dk), torch.float32)
    _need("last_accepted", last_accepted, (B,), torch.int32)
    if path_out is not None:
        _need("path_out", path_out, (B, N), torch.int32)
    if path_len_out is not None:
        _need("path_len_out", path_len_out, (B,), torch.int32)
    if dev_status is not None:
        _need("dev_status", dev_status, (B,), torch.int32)
    _raise_on(lib().gdn_commit_path(B, N, H, dk, dv, factors.qkv_dtype, _p(S), _p(factors.buf),
                                    _p(last_accepted), _p(path_out), _p(path_len_out),
                                    _p(dev_status), _stream(stream)))


# ---------------------------------------------------------------------------
# layer scaffold (gdnlayer.h)
# ---------------------------------------------------------------------------

def _need_rows(name, t, dtype):
    """A 2-D (or more) tensor on the GPU whose rows are contiguous; returns (rows, cols, ld)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with contiguous rows")
    return t.shape[0], t.shape[1], t.stride(0)


def gdn_linear(A, W, C=None, R=None, C_bf16=None, w_layout: int = GDN_W_ROWS,
               stream=None) -> None:
    """C = A W^T (+ R); see ``gdn_linear`` in gdnlayer.h.  A [M][K] bf16; W bf16
    [Nc][K] (GDN_W_ROWS) or its gdn_pack_weights image (GDN_W_PACKED, same shape)."""
    M, K = A.shape
    Nc = W.shape[0]
    _need("A", A, (M, K), torch.bfloat16)
    _need("W", W, (Nc, K), torch.bfloat16)
    if R is not None:
        _need("R", R, (M, Nc), torch.float32)
    if C is not None:
        _need("C", C, (M, Nc), torch.float32)
    if C_bf16 is not None:
        _need("C_bf16", C_bf16, (M, Nc), torch.bfloat16)
    _raise_on(lib().gdn_linear(M, Nc, K, _p(A), _p(W), int(w_layout), _p(R), _p(C),
                               _p(C_bf16), _stream(stream)))


def gdn_pack_weights(W, W_packed, stream=None) -> None:
    """Reorder bf16 W [Nc][K] into the GDN_W_PACKED layout (same shape, other buffer)."""
    Nc, K = W.shape
    _need("W", W, (Nc, K), torch.bfloat16)
    _need("W_packed", W_packed, (Nc, K), torch.bfloat16)
    _raise_on(lib().gdn_pack_weights(Nc, K, _p(W), _p(W_packed), _stream(stream)))


def gdn_layer_prep(P, x, W_ab, parents, conv_w, hist, q, k, v, beta, g,
                   gate_shift: float = 2.0, stream=None) -> None:
    """Convolution along root paths, SiLU, L2 norm, beta and g; see gdnlayer.h.
    P [B][N][2H(dk+dv)] FP32, x [B][N][D] bf16, W_ab [2H][D] bf16."""
    if q.dim() != 4:
        raise ValueError("q must be [B][N][H][dk]")
    B, N, H, dk = q.shape
    dv = v.shape[-1]
    D = x.shape[-1]
    Cc = H * (2 * dk + dv)
    _need("P", P, (B, N, 2 * H * (dk + dv)), torch.float32)
    _need("x", x, (B, N, D), torch.bfloat16)
    _need("W_ab", W_ab, (2 * H, D), torch.bfloat16)
    _need("parents", parents, (B, N), torch.int32)
    _need("conv_w", conv_w, (Cc, 4), torch.float32)
    _need("hist", hist, (B, 3, Cc), torch.float32)
    _need("q", q, (B, N, H, dk), torch.bfloat16)
    _need("k", k, (B, N, H, dk), torch.bfloat16)
    _need("v", v, (B, N, H, dv), torch.bfloat16)
    _need("beta", beta, (B, N, H), torch.float32)
    _need("g", g, (B, N, H), torch.float32)
    _raise_on(lib().gdn_layer_prep(B, N, H, dk, dv, D, _p(P), _p(x), _p(W_ab), _p(parents),
                                   _p(conv_w), _p(hist), float(gate_shift), _p(q), _p(k), _p(v),
                                   _p(beta), _p(g), _stream(stream)))


def gdn_layer_prep_delayed(P, x, W_ab, parents, conv_w, hist, q, k, v, beta, g, P_prev,
                           parents_prev, last_prev, hist_out, gate_shift: float = 2.0,
                           dev_status=None, stream=None) -> None:
    """gdn_conv_commit of the previous step's accepted path (into hist_out) and
    gdn_layer_prep from the result, in one launch; see gdnlayer.h."""
    if q.dim() != 4:
        raise ValueError("q must be [B][N][H][dk]")
    B, N, H, dk = q.shape
    dv = v.shape[-1]
    D = x.shape[-1]
    Cc = H * (2 * dk + dv)
    Np = parents_prev.shape[-1]
    _need("P", P, (B, N, 2 * H * (dk + dv)), torch.float32)
    _need("x", x, (B, N, D), torch.bfloat16)
    _need("W_ab", W_ab, (2 * H, D), torch.bfloat16)
    _need("parents", parents, (B, N), torch.int32)
    _need("conv_w", conv_w, (Cc, 4), torch.float32)
    _need("hist", hist, (B, 3, Cc), torch.float32)
    _need("q", q, (B, N, H, dk), torch.bfloat16)
    _need("k", k, (B, N, H, dk), torch.bfloat16)
    _need("v", v, (B, N, H, dv), torch.bfloat16)
    _need("beta", beta, (B, N, H), torch.float32)
    _need("g", g, (B, N, H), torch.float32)
    _need("P_prev", P_prev, (B, Np, 2 * H * (dk + dv)), torch.float32)
    _need("parents_prev", parents_prev, (B, Np), torch.int32)
    _need("last_prev", last_prev, (B,), torch.int32)
    _need("hist_out", hist_out, (B, 3, Cc), torch.float32)
    if dev_status is not None:
        _need("dev_status", dev_status, (B,), torch.int32)
    _raise_on(lib().gdn_layer_prep_delayed(
        B, Np, N, H, dk, dv, D, _p(P), _p(x), _p(W_ab), _p(parents), _p(conv_w), _p(hist),
        float(gate_shift), _p(q), _p(k), _p(v), _p(beta), _p(g), _p(P_prev), _p(parents_prev),
        _p(last_prev), _p(hist_out), _p(dev_status), _stream(stream)))


def gdn_gate_merge(o, gate, Y, stream=None) -> None:
    """Y = bf16(o * SiLU(gate)); o [M][Cw] FP32, gate a row-strided [M][Cw] FP32 view."""
    M, Cw = o.shape
    _need("o", o, (M, Cw), torch.float32)
    _need("Y", Y, (M, Cw), torch.bfloat16)
    gm, gc, ldg = _need_rows("gate", gate, torch.float32)
    if (gm, gc) != (M, Cw):
        raise ValueError(f"gate has shape {(gm, gc)}, expected {(M, Cw)}")
    _raise_on(lib().gdn_gate_merge(M, Cw, _p(o), _p(gate), ldg, _p(Y), _stream(stream)))


def gdn_layer_verify(S, parents, q, k, v, beta, g, gate, Y, factors: FactorRecord,
                     prev_factors: FactorRecord = None, last_accepted=None, scale: float = 1.0,
                     commit_status=None, dev_status=None, stream=None) -> None:
    """Tree verification (delayed when prev_factors is given) writing
    Y = bf16(O * SiLU(gate)) instead of O; see ``gdn_layer_verify`` in gdnlayer.h.
    gate is a row-strided [B*N][H*dv] FP32 view (the gate block of P)."""
    B, N, H, dk, dv, code = _check_draft(S, q, k, v, beta, g)
    if code != GDN_BF16:
        raise TypeError("gdn_layer_verify takes bf16 q, k, v")
    _need("parents", parents, (B, N), torch.int32)
    _need("Y", Y, (B * N, H * dv), torch.bfloat16)
    gm, gc, ldg = _need_rows("gate", gate, torch.float32)
    if (gm, gc) != (B * N, H * dv):
        raise ValueError(f"gate has shape {(gm, gc)}, expected {(B * N, H * dv)}")
    _check_record(factors, B, N, H, dk, dv, code)
    n_prev = 0
    if prev_factors is not None:
        pf = prev_factors
        if (pf.B, pf.H, pf.dk, pf.dv, pf.qkv_dtype) != (B, H, dk, dv, code):
            raise ValueError("prev_factors sizes do not match the call")
        _need("last_accepted", last_accepted, (B,), torch.int32)
        n_prev = pf.N
    for name, t in (("commit_status", commit_status), ("dev_status", dev_status)):
        if t is not None:
            _need(name, t, (B,), torch.int32)
    _raise_on(lib().gdn_layer_verify(
        B, n_prev, N, H, dk, dv, _p(S), _p(prev_factors.buf if prev_factors is not None else None),
        _p(last_accepted), _p(commit_status), _p(parents), _p(q), _p(k), _p(v), _p(beta), _p(g),
        float(scale), _p(gate), ldg, _p(Y), _p(factors.buf), _p(dev_status), _stream(stream)))


def gdn_conv_commit(P, parents, last_accepted, hist, dev_status=None, stream=None) -> None:
    """Shift the accepted path's convolution inputs into hist; see gdnlayer.h."""
    B, N = parents.shape
    Cc = hist.shape[-1]
    _need("parents", parents, (B, N), torch.int32)
    _need("last_accepted", last_accepted, (B,), torch.int32)
    _need("hist", hist, (B, 3, Cc), torch.float32)
    if P.dim() != 3 or tuple(P.shape[:2]) != (B, N) or not P.is_contiguous():
        raise ValueError("P must be a contiguous [B][N][ldP] tensor")
    if P.dtype != torch.float32 or P.device.type != "cuda":
        raise TypeError("P must be a float32 GPU tensor")
    if dev_status is not None:
        _need("dev_status", dev_status, (B,), torch.int32)
    _raise_on(lib().gdn_conv_commit(B, N, Cc, _p(P), P.shape[2], _p(parents), _p(last_accepted),
                                    _p(hist), _p(dev_status), _stream(stream)))


def gdn_decode_step(S, q, k, v, beta, g, out, scale: float = 1.0, stream=None) -> None:
    """One token of the recurrence, S updated in place; see ``gdn_decode_step``."""
    if S.dim() != 4:
        raise ValueError("S must be [B][H][dv][dk]")
    B, H, dv, dk = S.shape
    dt = q.dtype
    _need("S", S, (B, H, dv, dk), torch.float32)
    _need("q", q, (B, H, dk), dt)
    _need("k", k, (B, H, dk), dt)
    _need("v", v, (B, H, dv), dt)
    _need("beta", beta, (B, H), torch.float32)
    _need("g", g, (B, H), torch.float32)
    _need("out", out, (B, H, dv), torch.float32)
    _raise_on(lib().gdn_decode_step(B, H, dk, dv, dtype_code(dt), _p(S), _p(q), _p(k), _p(v),
                                    _p(beta), _p(g), float(scale), _p(out), _stream(stream)))


# ---------------------------------------------------------------------------
# gdnnext.h
# ---------------------------------------------------------------------------

def gdn_replay_verify(S0, parents, q, k, v, beta, g, ends, out, scale: float = 1.0,
                      dev_status=None, stream=None) -> None:
    """Root-to-leaf replay of the paths ending at ``ends`` [B][P]; see
    ``gdn_replay_verify`` in gdnnext.h."""
    B, N, H, dk, dv, code = _check_draft(S0, q, k, v, beta, g)
    _need("parents", parents, (B, N), torch.int32)
    if ends.dim() != 2:
        raise ValueError("ends must be [B][P]")
    _need("ends", ends, (B, ends.shape[1]), torch.int32)
    _need("out", out, (B, N, H, dv), torch.float32)
    if dev_status is not None:
        _need("dev_status", dev_status, (B,), torch.int32)
    _raise_on(lib().gdn_replay_verify(B, N, H, dk, dv, code, _p(S0), _p(parents), _p(q), _p(k),
                                      _p(v), _p(beta), _p(g), float(scale), _p(ends),
                                      int(ends.shape[1]), _p(out), _p(dev_status),
                                      _stream(stream)))


def gdn_replay_commit(S, parents, k, v, beta, g, last_accepted, dev_status=None,
                      stream=None) -> None:
    """Token replay of the accepted path into S (in place); see
    ``gdn_replay_commit`` in gdnnext.h."""
    if S.dim() != 4 or k.dim() != 4:
        raise ValueError("S must be [B][H][dv][dk] and k [B][N][H][dk]")
    B, H, dv, dk = S.shape
    N = k.shape[1]
    dt = k.dtype
    _need("S", S, (B, H, dv, dk), torch.float32)
    _need("parents", parents, (B, N), torch.int32)
    _need("k", k, (B, N, H, dk), dt)
    _need("v", v, (B, N, H, dv), dt)
    _need("beta", beta, (B, N, H), torch.float32)
    _need("g", g, (B, N, H), torch.float32)
    _need("last_accepted", last_accepted, (B,), torch.int32)
    if dev_status is not None:
        _need("dev_status", dev_status, (B,), torch.int32)
    _raise_on(lib().gdn_replay_commit(B, N, H, dk, dv, dtype_code(dt), _p(S), _p(parents),
                                      _p(k), _p(v), _p(beta), _p(g), _p(last_accepted),
                                      _p(dev_status), _stream(stream)))


class HybridPlan:
    """gdn_hybrid_plan's result: the plan on the device and its level sizes on
    the host."""

    def __init__(self, parents_host, device="cuda"):
        import numpy as np
        par = np.ascontiguousarray(parents_host, dtype=np.int32)
        if par.ndim != 2:
            raise ValueError("parents must be [B][N]")
        B, N = par.shape
        n = int(lib().gdn_hybrid_plan_entries(B, N))
        if n == 0:
            raise GdnError(GDN_ERR_SHAPE, f"unsupported plan sizes B={B} N={N}")
        plan = np.empty(n, dtype=np.int32)
        cpl = np.zeros(N, dtype=np.int32)
        lev = np.zeros(1, dtype=np.int32)
        _raise_on(lib().gdn_hybrid_plan(B, N, par.ctypes.data_as(ctypes.c_void_p),
                                        plan.ctypes.data_as(ctypes.c_void_p),
                                        cpl.ctypes.data_as(ctypes.c_void_p),
                                        lev.ctypes.data_as(ctypes.c_void_p)))
        self.B, self.N = B, N
        self.levels = int(lev[0])
        self.chains_per_level = cpl  # host, kept alive for the launches
        self.plan_host = plan
        self.plan = torch.from_numpy(plan).to(device)


def gdn_hybrid_verify(S0, parents, q, k, v, beta, g, out, factors: FactorRecord,
                      plan: HybridPlan, scale: float = 1.0, dev_status=None,
                      stream=None) -> None:
    """Chain-decomposed hybrid verification; see ``gdn_hybrid_verify`` in gdnnext.h."""
    B, N, H, dk, dv, code = _check_draft(S0, q, k, v, beta, g)
    _need("parents", parents, (B, N), torch.int32)
    _need("out", out, (B, N, H, dv), torch.float32)
    _check_record(factors, B, N, H, dk, dv, code)
    if (plan.B, plan.N) != (B, N):
        raise ValueError("the plan was made for other sizes")
    if dev_status is not None:
        _need("dev_status", dev_status, (B,), torch.int32)
    _raise_on(lib().gdn_hybrid_verify(
        B, N, H, dk, dv, code, _p(S0), _p(parents), _p(q), _p(k), _p(v), _p(beta), _p(g),
        float(scale), _p(out), _p(factors.buf), _p(plan.plan), plan.levels,
        plan.chains_per_level.ctypes.data_as(ctypes.c_void_p), _p(dev_status),
        _stream(stream)))


def gdn_prune_draft(parents, conf, tau: float, kept, new_parents, count, dev_status=None,
                    stream=None) -> None:
    """Confidence-guided pruning of candidate trees [B][M] to at most T = kept.shape[1]
    nodes; see ``gdn_prune_draft`` in gdnnext.h."""
    if parents.dim() != 2 or kept.dim() != 2:
        raise ValueError("parents must be [B][M] and kept [B][T]")
    B, M = parents.shape
    T = kept.shape[1]
    _need("parents", parents, (B, M), torch.int32)
    _need("conf", conf, (B, M), torch.float32)
    _need("kept", kept, (B, T), torch.int32)
    _need("new_parents", new_parents, (B, T), torch.int32)
    _need("count", count, (B,), torch.int32)
    if dev_status is not None:
        _need("dev_status", dev_status, (B,), torch.int32)
    _raise_on(lib().gdn_prune_draft(B, M, T, float(tau), _p(parents), _p(conf), _p(kept),
                                    _p(new_parents), _p(count), _p(dev_status), _stream(stream)))
