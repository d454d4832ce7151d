"""Blockwise-FP8 MoE FFN forward for AMD MI355X (gfx950): Python binding.

The binding only marshals arguments: it allocates outputs with torch (device
memory), passes raw pointers and torch's current HIP stream to libmoefp8.so,
and raises MoeError on a non-zero status.  Every step of the layer runs in the
library's HIP kernels; there is no fallback when the library is missing.

Calls (same names as the C ABI in include/moefp8.h):
    fp8_quant_1x128, fp8_quant_128x128, fp8_rmsnorm_quant_1x128, moe_pack_weights, moe_route,
    moe_bias_update, moe_permute, moe_unpermute, fp8_grouped_gemm_blockscaled, moe_ffn_workspace_size,
    moe_ffn_forward, moe_ffn_forward_noalloc, moe_padded_rows, fp8_quant_128x1_grouped,
    moe_pack_weights_transposed, fp8_grouped_gemm_wgrad, moe_validation_enabled

With MOEFP8_VALIDATE set in the environment, the calls check the device data they read (ids,
positions, offsets, given scores) before launching and raise MoeError with status
MOE_ERR_INVALID_DATA when an element breaks the call's contract.
"""
from __future__ import annotations

import ctypes
import dataclasses

import torch

from . import _lib
from ._lib import (MOE_ERR_INVALID_DATA, MOE_EPI_STORE_BF16, MOE_EPI_STORE_F32, MOE_EPI_SWIGLU_QUANT,  # noqa: F401
                   MOE_EPI_WEIGHTED_SCATTER_ADD, MOE_FWD_DETERMINISTIC, MOE_GROUP_SCORE_MAX,
                   MOE_GROUP_SCORE_TOP2_SUM, MOE_ROUTE_SCORES_GIVEN, MOE_SCALE_F32, MOE_SCALE_UE8M0)


def _fmt(ue8m0: bool) -> int:
    return MOE_SCALE_UE8M0 if ue8m0 else MOE_SCALE_F32


class MoeError(RuntimeError):
    def __init__(self, call: str, status: int, msg: str):
        super().__init__(f"{call}: {msg} ({status})")
        self.status = status


def _check(call: str, status: int) -> None:
    if status != 0:
        lib = _lib.load()
        raise MoeError(call, status, f"{lib.moe_status_string(status).decode()}: {lib.moe_last_error().decode()}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@dataclasses.dataclass(frozen=True)
class MoeConfig:
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    n_shared: int
    inter_shared: int
    n_group: int
    topk_group: int
    group_score: int = MOE_GROUP_SCORE_TOP2_SUM
    routed_scale: float = 1.0
    ue8m0: bool = False                 # power-of-two activation scales (weights quantised the same way)
    norm_eps: float = 1e-6              # RMSNorm epsilon, used when MoeWeights.norm_w is set

    def c(self) -> _lib.MoeCfgC:
        return _lib.MoeCfgC(self.hidden, self.inter, self.n_experts, self.top_k, self.n_shared, self.inter_shared,
                            self.n_group, self.topk_group, self.group_score, self.routed_scale, _fmt(self.ue8m0),
                            self.norm_eps)

    @staticmethod
    def of(shape, **kw) -> "MoeConfig":
        """From any object with the layer's shape fields (hidden, inter, n_experts, ...)."""
        return MoeConfig(shape.hidden, shape.inter, shape.n_experts, shape.top_k, shape.n_shared, shape.inter_shared,
                         shape.n_group, shape.topk_group, MOE_GROUP_SCORE_TOP2_SUM, float(shape.routed_scale), **kw)


@dataclasses.dataclass
class MoeWeights:
    """Device tensors of one layer (see moe_weights_t): codes uint8, scales fp32, router bf16."""
    w13_q: torch.Tensor | None = None
    w13_s: torch.Tensor | None = None
    w2_q: torch.Tensor | None = None
    w2_s: torch.Tensor | None = None
    sh_w13_q: torch.Tensor | None = None
    sh_w13_s: torch.Tensor | None = None
    sh_w2_q: torch.Tensor | None = None
    sh_w2_s: torch.Tensor | None = None
    w_router: torch.Tensor | None = None
    bias: torch.Tensor | None = None
    norm_w: torch.Tensor | None = None   # bf16 [hidden]: RMSNorm applied to x first

    def c(self) -> _lib.MoeWeightsC:
        f = {n: (None if getattr(self, n) is None else getattr(self, n).data_ptr()) for n in
             ("w_router", "bias", "w13_q", "w13_s", "w2_q", "w2_s", "sh_w13_q", "sh_w13_s", "sh_w2_q", "sh_w2_s",
              "norm_w")}
        return _lib.MoeWeightsC(**f)


def fp8_quant_1x128(x: torch.Tensor, q: torch.Tensor | None = None, s: torch.Tensor | None = None,
                    ue8m0: bool = False):
    """x [rows, cols] bf16 or fp32 -> (codes uint8 [rows, cols], scales fp32 [rows, cols/128])."""
    _dev(x, "x")
    rows, cols = x.shape
    dt = {torch.bfloat16: _lib.MOE_DTYPE_BF16, torch.float32: _lib.MOE_DTYPE_F32}.get(x.dtype)
    if dt is None:
        raise ValueError("x must be bfloat16 or float32")
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device) if q is None else q
    s = torch.empty((rows, max(cols // 128, 0)), dtype=torch.float32, device=x.device) if s is None else s
    _check("fp8_quant_1x128", _lib.load().fp8_quant_1x128(_p(x), dt, rows, cols, cols, _p(q), cols, _p(s),
                                                          _fmt(ue8m0), _stream(x)))
    return q, s


def fp8_quant_128x128(w: torch.Tensor, q: torch.Tensor | None = None, s: torch.Tensor | None = None,
                      ue8m0: bool = False):
    """w [rows, cols] fp32 -> (codes uint8 [rows, cols], scales fp32 [rows/128, cols/128])."""
    _dev(w, "w")
    rows, cols = w.shape
    if w.dtype != torch.float32:
        raise ValueError("w must be float32")
    q = torch.empty((rows, cols), dtype=torch.uint8, device=w.device) if q is None else q
    s = torch.empty((rows // 128, cols // 128), dtype=torch.float32, device=w.device) if s is None else s
    _check("fp8_quant_128x128", _lib.load().fp8_quant_128x128(_p(w), rows, cols, _p(q), _p(s), _fmt(ue8m0),
                                                              _stream(w)))
    return q, s


def fp8_rmsnorm_quant_1x128(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6, want_y: bool = True,
                            ue8m0: bool = False):
    """x bf16 [rows, cols], gamma bf16 [cols] -> (y bf16 [rows, cols] or None, codes uint8, scales fp32)."""
    _dev(x, "x")
    _dev(gamma, "gamma")
    if x.dtype != torch.bfloat16 or gamma.dtype != torch.bfloat16:
        raise ValueError("x and gamma must be bfloat16")
    rows, cols = x.shape
    y = torch.empty_like(x) if want_y else None
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    s = torch.empty((rows, max(cols // 128, 0)), dtype=torch.float32, device=x.device)
    _check("fp8_rmsnorm_quant_1x128", _lib.load().fp8_rmsnorm_quant_1x128(
        _p(x), _p(gamma), eps, rows, cols, cols, _p(y), cols, _p(q), cols, _p(s), _fmt(ue8m0), _stream(x)))
    return y, q, s


def moe_bias_update(topk_idx: torch.Tensor, n_experts: int, gamma: float, bias: torch.Tensor,
                    counts: torch.Tensor | None = None) -> torch.Tensor | None:
    """In place: bias[e] += gamma * sign(mean load - load_e) from int32 topk_idx [T, k].  Fills and
    returns ``counts`` (int32 [E]) when given."""
    _dev(topk_idx, "topk_idx")
    _dev(bias, "bias")
    T, k = topk_idx.shape
    _check("moe_bias_update", _lib.load().moe_bias_update(_p(topk_idx), T, k, n_experts, gamma, _p(bias), _p(counts),
                                                          _stream(bias)))
    return counts


def moe_pack_weights(w_q: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Row-major e4m3 codes [N, K] or [G, N, K] (uint8) -> the MFMA-fragment order the GEMMs read
    (same shape and size; see moe_pack_weights in the C header)."""
    _dev(w_q, "w_q")
    G, N, K = (1, *w_q.shape) if w_q.dim() == 2 else tuple(w_q.shape)
    out = torch.empty_like(w_q) if out is None else out
    _check("moe_pack_weights", _lib.load().moe_pack_weights(_p(w_q), G, N, K, _p(out), _stream(w_q)))
    return out


def quantize_pack_128x128(w: torch.Tensor, q: torch.Tensor | None = None, s: torch.Tensor | None = None,
                          ue8m0: bool = False):
    """fp32 weights [N, K] -> (packed e4m3 codes [N, K], scales [N/128, K/128]): fp8_quant_128x128
    followed by moe_pack_weights (a temporary holds the row-major codes)."""
    rm, s = fp8_quant_128x128(w, s=s, ue8m0=ue8m0)
    return moe_pack_weights(rm, out=q), s


def moe_route(cfg: MoeConfig, T: int, device, scores: torch.Tensor | None = None, x: torch.Tensor | None = None,
              w_router: torch.Tensor | None = None, bias: torch.Tensor | None = None):
    """Gating.  With ``scores`` given, routes those; else computes sigmoid(x w_router^T) into a new
    scores tensor.  Returns (scores fp32 [T, E], topk_idx int32 [T, k], topk_w fp32 [T, k])."""
    given = scores is not None
    if not given:
        scores = torch.empty((T, cfg.n_experts), dtype=torch.float32, device=device)
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=device)
    w = torch.empty((T, cfg.top_k), dtype=torch.float32, device=device)
    c = cfg.c()
    _check("moe_route", _lib.load().moe_route(_p(x), _p(w_router), _p(bias), T, ctypes.byref(c), _p(scores),
                                              _lib.MOE_ROUTE_SCORES_GIVEN if given else 0, _p(idx), _p(w),
                                              _stream(scores)))
    return scores, idx, w


def moe_permute(topk_idx: torch.Tensor, n_experts: int, rows: torch.Tensor | None = None):
    """topk_idx int32 [T, k] -> (offsets [E+1], sorted_assign [T*k], assign_pos [T*k], gathered rows or None).
    ``rows`` (uint8 [T, row_bytes], row_bytes % 16 == 0) is gathered into sorted order when given."""
    _dev(topk_idx, "topk_idx")
    T, k = topk_idx.shape
    dev = topk_idx.device
    lib = _lib.load()
    offsets = torch.empty(n_experts + 1, dtype=torch.int32, device=dev)
    sa = torch.empty(T * k, dtype=torch.int32, device=dev)
    ap = torch.empty(T * k, dtype=torch.int32, device=dev)
    ws_bytes = lib.moe_permute_workspace_size(T, k, n_experts)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    out_rows = None
    row_bytes = 0
    if rows is not None:
        _dev(rows, "rows")
        row_bytes = rows.shape[1] * rows.element_size()
        out_rows = torch.empty((T * k,) + tuple(rows.shape[1:]), dtype=rows.dtype, device=dev)
    _check("moe_permute", lib.moe_permute(_p(topk_idx), T, k, n_experts, _p(offsets), _p(sa), _p(ap), _p(rows),
                                          row_bytes, _p(out_rows), _p(ws), ws_bytes, _stream(topk_idx)))
    return offsets, sa, ap, out_rows


def moe_unpermute(y_sorted: torch.Tensor, assign_pos: torch.Tensor, top_k: int, topk_w: torch.Tensor | None = None,
                  shared_y: torch.Tensor | None = None) -> torch.Tensor:
    """Without topk_w: [T*k, d] -> [T, k, d] (same dtype).  With topk_w (y fp32): the weighted
    combine (+ shared_y) -> bf16 [T, d]."""
    _dev(y_sorted, "y_sorted")
    n, d = y_sorted.shape
    T = n // top_k
    dt = {torch.float32: _lib.MOE_DTYPE_F32, torch.bfloat16: _lib.MOE_DTYPE_BF16, torch.uint8: _lib.MOE_DTYPE_U8}[
        y_sorted.dtype]
    if topk_w is None:
        out = torch.empty((T, top_k, d), dtype=y_sorted.dtype, device=y_sorted.device)
    else:
        out = torch.empty((T, d), dtype=torch.bfloat16, device=y_sorted.device)
    _check("moe_unpermute", _lib.load().moe_unpermute(_p(y_sorted), dt, _p(assign_pos), _p(topk_w), _p(shared_y), T,
                                                      top_k, d, _p(out), _stream(y_sorted)))
    return out


def fp8_grouped_gemm_blockscaled(a_q, a_s, b_q, b_s, offsets, epilogue: int, a_gather=None, m_max: int | None = None,
                                 out=None, h_s=None, dst_row=None, row_weight=None, out_rows: int | None = None,
                                 ue8m0: bool = False):
    """Grouped block-scaled GEMM (see the C header).  b_q uint8 [G, N, K].  Returns the output
    tensor (and h_s for MOE_EPI_SWIGLU_QUANT)."""
    G, N, K = b_q.shape
    M = int(m_max if m_max is not None else (a_gather.shape[0] if a_gather is not None else a_q.shape[0]))
    dev = a_q.device
    if out is None:
        if epilogue == MOE_EPI_SWIGLU_QUANT:
            out = torch.empty((M, N // 2), dtype=torch.uint8, device=dev)
        elif epilogue == MOE_EPI_STORE_BF16:
            out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        elif epilogue == MOE_EPI_WEIGHTED_SCATTER_ADD:
            out = torch.zeros((out_rows if out_rows is not None else M, N), dtype=torch.float32, device=dev)
        else:
            out = torch.empty((M, N), dtype=torch.float32, device=dev)
    if epilogue == MOE_EPI_SWIGLU_QUANT and h_s is None:
        h_s = torch.empty((M, N // 256), dtype=torch.float32, device=dev)
    epi = _lib.MoeEpiC(None if h_s is None else h_s.data_ptr(), None if dst_row is None else dst_row.data_ptr(),
                       None if row_weight is None else row_weight.data_ptr(), _fmt(ue8m0))
    _check("fp8_grouped_gemm_blockscaled", _lib.load().fp8_grouped_gemm_blockscaled(
        _p(a_q), _p(a_s), _p(a_gather), _p(b_q), _p(b_s), _p(offsets), G, M, N, K, epilogue, ctypes.byref(epi),
        _p(out), _stream(a_q)))
    return (out, h_s) if epilogue == MOE_EPI_SWIGLU_QUANT else out


def moe_ffn_workspace_size(T: int, cfg: MoeConfig) -> int:
    c = cfg.c()
    return int(_lib.load().moe_ffn_workspace_size(T, ctypes.byref(c)))


def alloc_workspace(T: int, cfg: MoeConfig, device) -> torch.Tensor:
    n = moe_ffn_workspace_size(T, cfg)
    if n == 0:
        raise ValueError("invalid configuration for moe_ffn_forward")
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_ffn_forward(x: torch.Tensor, cfg: MoeConfig, weights: MoeWeights, workspace: torch.Tensor | None = None,
                    out: torch.Tensor | None = None, scores: torch.Tensor | None = None, scores_given: bool = False,
                    topk_idx: torch.Tensor | None = None, topk_w: torch.Tensor | None = None,
                    deterministic: bool = False) -> torch.Tensor:
    """One layer: x bf16 [T, hidden] -> bf16 [T, hidden].  Optional scores / topk_idx / topk_w
    tensors receive the routing (with ``scores_given`` the scores are read instead)."""
    _dev(x, "x")
    T = x.shape[0]
    if workspace is None:
        workspace = alloc_workspace(T, cfg, x.device)
    out = torch.empty_like(x) if out is None else out
    c = cfg.c()
    wc = weights.c()
    flags = (_lib.MOE_ROUTE_SCORES_GIVEN if scores_given else 0) | (MOE_FWD_DETERMINISTIC if deterministic else 0)
    _check("moe_ffn_forward", _lib.load().moe_ffn_forward(
        _p(x), T, ctypes.byref(c), ctypes.byref(wc), _p(workspace), workspace.numel(), _p(out), _p(scores),
        _p(topk_idx), _p(topk_w), flags, _stream(x)))
    return out


def moe_ffn_forward_noalloc(x: torch.Tensor, cfg: MoeConfig, weights: MoeWeights, out: torch.Tensor | None = None,
                            scores: torch.Tensor | None = None, scores_given: bool = False,
                            topk_idx: torch.Tensor | None = None, topk_w: torch.Tensor | None = None,
                            deterministic: bool = False) -> torch.Tensor:
    """moe_ffn_forward with the library's static device workspace (no workspace argument; the
    library allocates nothing).  Raises MoeError (MOE_ERR_WORKSPACE) when T needs more than
    MOE_NOALLOC_SCRATCH_BYTES of workspace.  Calls on one GPU share the array: do not overlap them."""
    _dev(x, "x")
    T = x.shape[0]
    out = torch.empty_like(x) if out is None else out
    c = cfg.c()
    wc = weights.c()
    flags = (_lib.MOE_ROUTE_SCORES_GIVEN if scores_given else 0) | (MOE_FWD_DETERMINISTIC if deterministic else 0)
    _check("moe_ffn_forward_noalloc", _lib.load().moe_ffn_forward_noalloc(
        _p(x), T, ctypes.byref(c), ctypes.byref(wc), _p(out), _p(scores), _p(topk_idx), _p(topk_w), flags,
        _stream(x)))
    return out


def moe_validation_enabled() -> bool:
    """Whether calls made now check their device data first (MOEFP8_VALIDATE, read per call)."""
    return bool(_lib.load().moe_validation_enabled())


# ---- FP8 backward of the grouped GEMMs ----

def moe_padded_rows(M: int, G: int) -> int:
    """Upper bound of the rows of M rows in G groups once every group is padded to 128 rows."""
    return int(_lib.load().moe_padded_rows(M, G))


def fp8_quant_128x1_grouped(x: torch.Tensor, offsets: torch.Tensor, ue8m0: bool = False):
    """x [M, N] bf16 or fp32, rows grouped by offsets int32 [G+1] -> (q_t uint8 [N, Mp], s_t fp32
    [N, Mp/128], padded offsets int32 [G+1]): 128x1 tiles per column and group, stored transposed
    (Mp = moe_padded_rows(M, G); columns past the padded rows are left unwritten)."""
    _dev(x, "x")
    _dev(offsets, "offsets")
    M, N = x.shape
    G = offsets.numel() - 1
    dt = {torch.bfloat16: _lib.MOE_DTYPE_BF16, torch.float32: _lib.MOE_DTYPE_F32}.get(x.dtype)
    if dt is None:
        raise ValueError("x must be bfloat16 or float32")
    mp = moe_padded_rows(M, G)
    q = torch.empty((N, mp), dtype=torch.uint8, device=x.device)
    s = torch.empty((N, mp // 128), dtype=torch.float32, device=x.device)
    po = torch.empty(G + 1, dtype=torch.int32, device=x.device)
    _check("fp8_quant_128x1_grouped", _lib.load().fp8_quant_128x1_grouped(
        _p(x), dt, M, N, N, _p(offsets), G, _p(po), _p(q), mp, _p(s), _fmt(ue8m0), _stream(x)))
    return q, s, po


def moe_pack_weights_transposed(w_q: torch.Tensor, w_s: torch.Tensor):
    """Row-major e4m3 W [G, N, K] (or [N, K]) with block scales [G, N/128, K/128] -> W^T in the
    GEMMs' fragment order [G, K, N] and its block scales [G, K/128, N/128]."""
    _dev(w_q, "w_q")
    _dev(w_s, "w_s")
    squeeze = w_q.dim() == 2
    G, N, K = (1, *w_q.shape) if squeeze else tuple(w_q.shape)
    wt_q = torch.empty((G, K, N), dtype=torch.uint8, device=w_q.device)
    wt_s = torch.empty((G, K // 128, N // 128), dtype=torch.float32, device=w_q.device)
    _check("moe_pack_weights_transposed", _lib.load().moe_pack_weights_transposed(
        _p(w_q), _p(w_s), G, N, K, _p(wt_q), _p(wt_s), _stream(w_q)))
    return (wt_q[0], wt_s[0]) if squeeze else (wt_q, wt_s)


def fp8_grouped_gemm_wgrad(a_t: torch.Tensor, a_ts: torch.Tensor, b_t: torch.Tensor, b_ts: torch.Tensor,
                           padded: torch.Tensor, M: int, out: torch.Tensor | None = None, ue8m0: bool = False):
    """out[g] = A_g^T-operand x B_g over group g's padded rows: a_t [Na, Mp], b_t [Nb, Mp] from
    fp8_quant_128x1_grouped (same grouping, M rows before padding) -> fp32 [G, Na, Nb]."""
    _dev(a_t, "a_t")
    _dev(b_t, "b_t")
    Na, ld = a_t.shape
    Nb = b_t.shape[0]
    G = padded.numel() - 1
    if out is None:
        out = torch.empty((G, Na, Nb), dtype=torch.float32, device=a_t.device)
    _check("fp8_grouped_gemm_wgrad", _lib.load().fp8_grouped_gemm_wgrad(
        _p(a_t), _p(a_ts), _p(b_t), _p(b_ts), _p(padded), G, M, Na, Nb, ld, _p(out), _fmt(ue8m0), _stream(a_t)))
    return out
