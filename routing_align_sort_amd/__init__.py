"""Python binding of the MI355X MoE FFN layer library (libmoe_mi355x.so).

Argument marshalling only: every step of the layer runs in the HIP kernels of
the C-ABI library declared in include/moe_mi355x.h.  Tensors are torch CUDA
(HIP) tensors; calls are enqueued on torch's current stream.  If the library
has not been built this module raises on first use -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB_PATH selects another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(_HERE, "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_SCRATCH_LIMIT = range(6)
MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_FP4_E2M1 = 0, 1, 2, 3
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1

_lib = None


class MoEError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


class _RouteParams(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("E", ctypes.c_int32), ("K", ctypes.c_int32),
                ("score", ctypes.c_int32), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("routed_scaling", ctypes.c_float), ("append_shared", ctypes.c_int32)]


class _FfnParams(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("K", ctypes.c_int32), ("E", ctypes.c_int32),
                ("H", ctypes.c_int32), ("I", ctypes.c_int32), ("B", ctypes.c_int32),
                ("w_dtype", ctypes.c_int32), ("x_dtype", ctypes.c_int32),
                ("weight_layout", ctypes.c_int32), ("row_layout", ctypes.c_int32),
                ("schedule", ctypes.c_int32), ("grad_dtype", ctypes.c_int32),
                ("y_dtype", ctypes.c_int32), ("x_quantized", ctypes.c_int32)]


EXPORTED = ("moe_abi_version", "moe_status_string", "moe_route_topk", "moe_align_sort_capacity",
            "moe_align_sort_workspace_bytes", "moe_align_sort", "moe_grouped_ffn_workspace_bytes",
            "moe_grouped_ffn", "moe_grouped_ffn_profiled", "moe_grouped_ffn_top1", "moe_prepack_weights",
            "moe_prepack_block_scales", "moe_combine", "moe_combine_slots", "moe_permute_rows", "moe_unpermute_combine",
            "moe_unpermute_combine_backward", "moe_ffn_backward_workspace_bytes", "moe_ffn_backward",
            "moe_grouped_ffn_train", "moe_route_backward", "moe_align_sort_noalloc",
            "moe_align_sort_noalloc_scratch_bytes", "moe_route_topk_quantize")


def load_library(path: str = LIB_PATH):
    """Load and type the C-ABI library (no GPU needed to load it)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m routing_align_sort_amd.build`")
    lib = ctypes.CDLL(path)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.moe_abi_version.restype = i32
    lib.moe_status_string.argtypes = [i32]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_route_topk.argtypes = [ctypes.POINTER(_RouteParams), P, P, P, P, P]
    lib.moe_route_topk.restype = i32
    lib.moe_route_topk_quantize.argtypes = [ctypes.POINTER(_RouteParams), P, P, P, P, ctypes.POINTER(_FfnParams),
                                            P, P, sz, P]
    lib.moe_route_topk_quantize.restype = i32
    lib.moe_align_sort_capacity.argtypes = [i32, i32, i32, i32]
    lib.moe_align_sort_capacity.restype = i64
    lib.moe_align_sort_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.moe_align_sort_workspace_bytes.restype = i64
    lib.moe_align_sort.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P, sz, P]
    lib.moe_align_sort.restype = i32
    lib.moe_align_sort_noalloc_scratch_bytes.argtypes = []
    lib.moe_align_sort_noalloc_scratch_bytes.restype = i64
    lib.moe_align_sort_noalloc.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P]
    lib.moe_align_sort_noalloc.restype = i32
    lib.moe_grouped_ffn_workspace_bytes.argtypes = [ctypes.POINTER(_FfnParams)]
    lib.moe_grouped_ffn_workspace_bytes.restype = i64
    lib.moe_grouped_ffn.argtypes = [ctypes.POINTER(_FfnParams), P, P, P, P, P, P, P, P, P, P, sz, P]
    lib.moe_grouped_ffn.restype = i32
    lib.moe_grouped_ffn_profiled.argtypes = [ctypes.POINTER(_FfnParams), P, P, P, P, P, P, P, P, P, P,
                                             sz, P, P]
    lib.moe_grouped_ffn_top1.argtypes = [ctypes.POINTER(_FfnParams), P, P, P, P, P, P, P, P, P, P, i32, P, P,
                                         sz, P]
    lib.moe_grouped_ffn_top1.restype = i32
    lib.moe_grouped_ffn_profiled.restype = i32
    lib.moe_prepack_weights.argtypes = [ctypes.POINTER(_FfnParams), P, P, P, P, P]
    lib.moe_prepack_weights.restype = i32
    lib.moe_prepack_block_scales.argtypes = [ctypes.POINTER(_FfnParams), P, P, P, P, P]
    lib.moe_prepack_block_scales.restype = i32
    lib.moe_combine.argtypes = [i32, i32, i32, i32, P, P, P, i32, P, P]
    lib.moe_combine.restype = i32
    lib.moe_combine_slots.argtypes = [i32, i32, i32, i32, P, i32, P, P, i32, P, P]
    lib.moe_combine_slots.restype = i32
    lib.moe_permute_rows.argtypes = [P, i32, i32, i32, i32, i64, P, P, P, P, P, P, P, P]
    lib.moe_permute_rows.restype = i32
    lib.moe_unpermute_combine.argtypes = [i32, i32, i32, P, P, P, i32, P, P]
    lib.moe_unpermute_combine.restype = i32
    lib.moe_unpermute_combine_backward.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P, i32, P, P, P]
    lib.moe_unpermute_combine_backward.restype = i32
    lib.moe_ffn_backward_workspace_bytes.argtypes = [ctypes.POINTER(_FfnParams)]
    lib.moe_ffn_backward_workspace_bytes.restype = i64
    lib.moe_ffn_backward.argtypes = [ctypes.POINTER(_FfnParams)] + [P] * 17 + [sz, P]
    lib.moe_grouped_ffn_train.argtypes = [ctypes.POINTER(_FfnParams)] + [P] * 8 + [P, sz, P]
    lib.moe_grouped_ffn_train.restype = i32
    lib.moe_ffn_backward.restype = i32
    lib.moe_route_backward.argtypes = [ctypes.POINTER(_RouteParams), P, P, P, P, P]
    lib.moe_route_backward.restype = i32
    _lib = lib
    return lib


def abi_version() -> int:
    return int(load_library().moe_abi_version())


def status_string(status: int) -> str:
    return load_library().moe_status_string(int(status)).decode()


def _check(fn, st):
    if st != MOE_OK:
        raise MoEError(fn, st)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, dtype, name, numel=None):
    if t.device.type != "cuda" or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous {dtype} tensor on the GPU, got "
                         f"{t.dtype} on {t.device} (contiguous={t.is_contiguous()})")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: expected {numel} elements, got {t.numel()}")


# ------------------------------------------------------------------ routing --
def moe_route_topk(logits, K, *, score="softmax", bias=None, n_group=1, topk_group=1,
                   renormalize=True, routed_scaling=1.0, append_shared=False,
                   topk_ids=None, topk_weights=None, stream=None):
    """Top-K routing of each row of fp32 ``logits`` [T,E]; returns (topk_ids, topk_weights)."""
    lib = load_library()
    T, E = logits.shape
    _need(logits, torch.float32, "logits")
    if bias is not None:
        _need(bias, torch.float32, "bias", E)
    KO = K + (1 if append_shared else 0)
    if topk_ids is None:
        topk_ids = torch.empty((T, KO), dtype=torch.int32, device=logits.device)
    if topk_weights is None:
        topk_weights = torch.empty((T, KO), dtype=torch.float32, device=logits.device)
    _need(topk_ids, torch.int32, "topk_ids", T * KO)
    _need(topk_weights, torch.float32, "topk_weights", T * KO)
    p = _RouteParams(T, E, K, {"softmax": 0, "sigmoid": 1}[score], n_group, topk_group,
                     int(bool(renormalize)), float(routed_scaling), int(bool(append_shared)))
    _check("moe_route_topk", lib.moe_route_topk(ctypes.byref(p), _ptr(logits), _ptr(bias),
                                                _ptr(topk_ids), _ptr(topk_weights), _stream(stream)))
    return topk_ids, topk_weights


def moe_route_topk_quantize(logits, K, x, workspace, *, w13, B, K_ffn=None, score="softmax", bias=None,
                            n_group=1, topk_group=1, renormalize=True, routed_scaling=1.0,
                            append_shared=False, fused=False, topk_ids=None, topk_weights=None, stream=None):
    """moe_route_topk, plus the per-token E4M3 quantisation of bf16 ``x`` into
    ``workspace`` (the moe_grouped_ffn workspace of E4M3 or MXFP4 weights
    ``w13`` at block size B), in one launch.  The FFN call that follows passes
    the same workspace with x_quantized=True.  K_ffn: slots per token of that
    FFN call (K, plus one with append_shared).  Returns (topk_ids, topk_weights)."""
    lib = load_library()
    T, E = logits.shape
    _need(logits, torch.float32, "logits")
    _need(x, torch.bfloat16, "x")
    if bias is not None:
        _need(bias, torch.float32, "bias", E)
    KO = K + (1 if append_shared else 0)
    if K_ffn is None:
        K_ffn = KO
    if topk_ids is None:
        topk_ids = torch.empty((T, KO), dtype=torch.int32, device=logits.device)
    if topk_weights is None:
        topk_weights = torch.empty((T, KO), dtype=torch.float32, device=logits.device)
    _need(topk_ids, torch.int32, "topk_ids", T * KO)
    _need(topk_weights, torch.float32, "topk_weights", T * KO)
    Ew, I, H = weight_dims(w13)
    if tuple(x.shape) != (T, H):
        raise ValueError("x must be [T, H]")
    rp = _RouteParams(T, E, K, {"softmax": 0, "sigmoid": 1}[score], n_group, topk_group,
                      int(bool(renormalize)), float(routed_scaling), int(bool(append_shared)))
    fp = _ffn_params(T, K_ffn, Ew, H, I, B, w13.dtype, torch.bfloat16, fused=fused, x_quantized=True)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("moe_route_topk_quantize", lib.moe_route_topk_quantize(
        ctypes.byref(rp), _ptr(logits), _ptr(bias), _ptr(topk_ids), _ptr(topk_weights), ctypes.byref(fp),
        _ptr(x), _ptr(workspace), ws_bytes, _stream(stream)))
    return topk_ids, topk_weights


# -------------------------------------------------------------- align&sort --
def moe_align_sort_capacity(T, K, E, B) -> int:
    c = int(load_library().moe_align_sort_capacity(T, K, E, B))
    if c < 0:
        raise MoEError("moe_align_sort_capacity", MOE_ERR_INVALID_ARG)
    return c


def moe_align_sort_workspace_bytes(T, K, E, B) -> int:
    c = int(load_library().moe_align_sort_workspace_bytes(T, K, E, B))
    if c < 0:
        raise MoEError("moe_align_sort_workspace_bytes", MOE_ERR_INVALID_ARG)
    return c


def moe_align_sort(topk_ids, E, B, *, sorted_token_ids=None, expert_ids=None,
                   num_tokens_post_padded=None, expert_offsets=None, workspace=None, stream=None):
    """Align & Sort of int32 ``topk_ids`` [T,K]; returns a dict of device tensors.

    A caller-given ``workspace`` must be zero-filled before its first use
    (every call leaves it so); without one a zeroed tensor is allocated."""
    lib = load_library()
    ids = topk_ids if topk_ids.dim() == 2 else topk_ids.view(-1, 1)
    T, K = ids.shape
    _need(ids, torch.int32, "topk_ids")
    dev = ids.device
    C = moe_align_sort_capacity(T, K, E, B)
    if sorted_token_ids is None:
        sorted_token_ids = torch.empty(C, dtype=torch.int32, device=dev)
    if expert_ids is None:
        expert_ids = torch.empty(C // B, dtype=torch.int32, device=dev)
    if num_tokens_post_padded is None:
        num_tokens_post_padded = torch.empty(1, dtype=torch.int32, device=dev)
    if expert_offsets is None:
        expert_offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    ws_need = moe_align_sort_workspace_bytes(T, K, E, B)
    if workspace is None and ws_need > 0:
        workspace = torch.zeros(ws_need, dtype=torch.uint8, device=dev)    # zero before its first use
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _need(sorted_token_ids, torch.int32, "sorted_token_ids", C)
    _need(expert_ids, torch.int32, "expert_ids", C // B)
    _need(num_tokens_post_padded, torch.int32, "num_tokens_post_padded", 1)
    _need(expert_offsets, torch.int32, "expert_offsets", E + 1)
    _check("moe_align_sort", lib.moe_align_sort(
        _ptr(ids), T, K, E, B, _ptr(sorted_token_ids), _ptr(expert_ids),
        _ptr(num_tokens_post_padded), _ptr(expert_offsets), _ptr(workspace), ws_bytes,
        _stream(stream)))
    return {"sorted_token_ids": sorted_token_ids, "expert_ids": expert_ids,
            "num_tokens_post_padded": num_tokens_post_padded, "expert_offsets": expert_offsets}


def moe_align_sort_noalloc_scratch_bytes() -> int:
    return int(load_library().moe_align_sort_noalloc_scratch_bytes())


def moe_align_sort_noalloc(topk_ids, E, B, *, sorted_token_ids, expert_ids, num_tokens_post_padded,
                           expert_offsets=None, stream=None):
    """moe_align_sort into caller-given outputs with no workspace: the library's
    fixed scratch stands in for it and nothing is allocated (outputs are
    required for that reason).  Calls that overlap on one device race."""
    lib = load_library()
    ids = topk_ids if topk_ids.dim() == 2 else topk_ids.view(-1, 1)
    T, K = ids.shape
    _need(ids, torch.int32, "topk_ids")
    C = moe_align_sort_capacity(T, K, E, B)
    _need(sorted_token_ids, torch.int32, "sorted_token_ids", C)
    _need(expert_ids, torch.int32, "expert_ids", C // B)
    _need(num_tokens_post_padded, torch.int32, "num_tokens_post_padded", 1)
    if expert_offsets is not None:
        _need(expert_offsets, torch.int32, "expert_offsets", E + 1)
    _check("moe_align_sort_noalloc", lib.moe_align_sort_noalloc(
        _ptr(ids), T, K, E, B, _ptr(sorted_token_ids), _ptr(expert_ids),
        _ptr(num_tokens_post_padded), _ptr(expert_offsets), _stream(stream)))
    return {"sorted_token_ids": sorted_token_ids, "expert_ids": expert_ids,
            "num_tokens_post_padded": num_tokens_post_padded, "expert_offsets": expert_offsets}


# -------------------------------------------------------------- grouped FFN --
_DT = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16, torch.float8_e4m3fn: MOE_FP8_E4M3,
       torch.float4_e2m1fn_x2: MOE_FP4_E2M1}
# MXFP4 weights are float4_e2m1fn_x2 tensors (one element = two E2M1 codes,
# the even column in the low nibble) with float8_e8m0fnu block scales, one per
# 32 elements of a row.
FP4 = torch.float4_e2m1fn_x2
E8M0 = torch.float8_e8m0fnu


def weight_dims(w13):
    """(E, I, H) of a gate/up weight tensor [E, 2I, H] (MXFP4: [E, 2I, H/2])."""
    E, I2, Hc = w13.shape
    return E, I2 // 2, Hc * (2 if w13.dtype == FP4 else 1)


MOE_LAYOUT_CANONICAL, MOE_LAYOUT_PACKED = 0, 1
MOE_ROWS_BY_TOKEN, MOE_ROWS_SORTED = 0, 1
MOE_SCHEDULE_TWO_LAUNCH, MOE_SCHEDULE_FUSED = 0, 1


def _ffn_params(T, K, E, H, I, B, w_dtype, x_dtype, packed=False, rows_sorted=False, fused=False,
                grad_dtype=torch.float32, y_dtype=torch.float32, x_quantized=False):
    return _FfnParams(T, K, E, H, I, B, _DT[w_dtype], _DT[x_dtype],
                      MOE_LAYOUT_PACKED if packed else MOE_LAYOUT_CANONICAL,
                      MOE_ROWS_SORTED if rows_sorted else MOE_ROWS_BY_TOKEN,
                      MOE_SCHEDULE_FUSED if fused else MOE_SCHEDULE_TWO_LAUNCH, _DT[grad_dtype],
                      _DT[y_dtype], int(bool(x_quantized)))


def moe_prepack_weights(w13, w2, *, stream=None):
    """One-time rewrite of canonical expert weights into the packed streaming
    layout; returns (w13_packed, w2_packed), same shapes and dtype (opaque)."""
    lib = load_library()
    E, I, H = weight_dims(w13)
    _need(w13, w13.dtype, "w13")
    _need(w2, w13.dtype, "w2", w13.numel() // 2)
    p13 = torch.empty_like(w13)
    p2 = torch.empty_like(w2)
    p = _ffn_params(1, 1, E, H, I, 16, w13.dtype, torch.bfloat16)
    _check("moe_prepack_weights", lib.moe_prepack_weights(ctypes.byref(p), _ptr(w13), _ptr(w2),
                                                          _ptr(p13), _ptr(p2), _stream(stream)))
    return p13, p2


def moe_prepack_block_scales(w13_scale, w2_scale, H, I, *, stream=None):
    """One-time rewrite of MXFP4 block scales (float8_e8m0fnu [E,2I,H/32] and
    [E,H,I/32]) into the order read beside packed weights; returns the pair."""
    lib = load_library()
    E = w13_scale.shape[0]
    _need(w13_scale, E8M0, "w13_scale", E * 2 * I * (H // 32))
    _need(w2_scale, E8M0, "w2_scale", E * H * (I // 32))
    p13 = torch.empty_like(w13_scale)
    p2 = torch.empty_like(w2_scale)
    p = _ffn_params(1, 1, E, H, I, 16, FP4, torch.bfloat16)
    _check("moe_prepack_block_scales", lib.moe_prepack_block_scales(
        ctypes.byref(p), _ptr(w13_scale), _ptr(w2_scale), _ptr(p13), _ptr(p2), _stream(stream)))
    return p13, p2


def moe_grouped_ffn_workspace_bytes(T, K, E, H, I, B, w_dtype, x_dtype, rows_sorted=False,
                                    fused=False) -> int:
    p = _ffn_params(T, K, E, H, I, B, w_dtype, x_dtype, rows_sorted=rows_sorted, fused=fused)
    c = int(load_library().moe_grouped_ffn_workspace_bytes(ctypes.byref(p)))
    if c < 0:
        raise MoEError("moe_grouped_ffn_workspace_bytes", MOE_ERR_UNSUPPORTED)
    return c


def moe_grouped_ffn(x, w13, w2, sorted_token_ids, expert_ids, num_tokens_post_padded, *, K, B,
                    w13_scale=None, w2_scale=None, y_slots=None, workspace=None, stream=None,
                    stage_events=None, packed=False, T=None, fused=False, y_dtype=None, x_quantized=False):
    """Grouped SwiGLU expert FFN over the sorted layout; returns y_slots [T*K, H],
    fp32, or bf16 (rounded to nearest even) with y_dtype=torch.bfloat16 or a
    bf16 y_slots given (not with fp32 weights or rows in the sorted order).

    With ``T`` given and x of C = capacity rows, x is taken in the sorted row
    order (as moe_permute_rows writes it) and the result is [C, H] in that
    order (row layout MOE_ROWS_SORTED).
    fused: both GEMMs in one persistent launch (schedule MOE_SCHEDULE_FUSED).
    stage_events: optional 5 raw hipEvent_t handles (ints) recorded at the stage
    boundaries (the profiling entry point).
    x_quantized: the workspace already holds x's E4M3 codes and scales from
    moe_route_topk_quantize (E4M3 / MXFP4 weights, rows by token)."""
    lib = load_library()
    rows_sorted = T is not None
    Tx, H = x.shape
    if not rows_sorted:
        T = Tx
    E, I, H2 = weight_dims(w13)
    fp4 = w13.dtype == FP4
    if H2 != H or tuple(w2.shape) != (E, H, I // 2 if fp4 else I):
        raise ValueError("weight shapes do not match x")
    _need(x, x.dtype, "x")
    _need(w13, w13.dtype, "w13")
    _need(w2, w13.dtype, "w2")
    for t, n in ((sorted_token_ids, "sorted_token_ids"), (expert_ids, "expert_ids"),
                 (num_tokens_post_padded, "num_tokens_post_padded")):
        _need(t, torch.int32, n)
    if w13.dtype == torch.float8_e4m3fn:
        _need(w13_scale, torch.float32, "w13_scale", E * 2 * I)
        _need(w2_scale, torch.float32, "w2_scale", E * H)
    if fp4:
        _need(w13_scale, E8M0, "w13_scale", E * 2 * I * (H // 32))
        _need(w2_scale, E8M0, "w2_scale", E * H * (I // 32))
    ny = T * K
    if rows_sorted:
        ny = moe_align_sort_capacity(T, K, E, B)
        if Tx != ny:
            raise ValueError(f"x in the sorted row order must have {ny} rows, got {Tx}")
    if y_dtype is None:
        y_dtype = y_slots.dtype if y_slots is not None else torch.float32
    if y_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("y_dtype must be float32 or bfloat16")
    if y_slots is None:
        y_slots = torch.empty((ny, H), dtype=y_dtype, device=x.device)
    _need(y_slots, y_dtype, "y_slots", ny * H)
    p = _ffn_params(T, K, E, H, I, B, w13.dtype, x.dtype, packed, rows_sorted, fused, y_dtype=y_dtype,
                    x_quantized=x_quantized)
    need = moe_grouped_ffn_workspace_bytes(T, K, E, H, I, B, w13.dtype, x.dtype, rows_sorted, fused)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    args = (ctypes.byref(p), _ptr(x), _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale),
            _ptr(sorted_token_ids), _ptr(expert_ids), _ptr(num_tokens_post_padded), _ptr(y_slots),
            _ptr(workspace), ws_bytes, _stream(stream))
    if stage_events is None:
        _check("moe_grouped_ffn", lib.moe_grouped_ffn(*args))
    else:
        ev = (ctypes.c_void_p * 5)(*stage_events)
        _check("moe_grouped_ffn_profiled", lib.moe_grouped_ffn_profiled(*args, ev))
    return y_slots


def moe_grouped_ffn_top1(x, w13, w2, sorted_token_ids, expert_ids, num_tokens_post_padded, topk_ids,
                         topk_weights, *, B, w13_scale=None, w2_scale=None, out_dtype=torch.bfloat16,
                         out=None, workspace=None, stream=None, packed=False, x_quantized=False):
    """moe_grouped_ffn + moe_combine for top-1 routing in one call: out[t] =
    w[t] * FFN(x[t]) (zero rows for ids outside [0,E)); same bits as the two calls."""
    lib = load_library()
    T, H = x.shape
    E, I, H2 = weight_dims(w13)
    fp4 = w13.dtype == FP4
    if H2 != H or tuple(w2.shape) != (E, H, I // 2 if fp4 else I):
        raise ValueError("weight shapes do not match x")
    if tuple(topk_ids.shape) != (T, 1):
        raise ValueError("moe_grouped_ffn_top1 needs topk_ids of shape [T, 1]")
    _need(x, x.dtype, "x")
    _need(w13, w13.dtype, "w13")
    _need(w2, w13.dtype, "w2")
    for t, n in ((sorted_token_ids, "sorted_token_ids"), (expert_ids, "expert_ids"),
                 (num_tokens_post_padded, "num_tokens_post_padded"), (topk_ids, "topk_ids")):
        _need(t, torch.int32, n)
    _need(topk_weights, torch.float32, "topk_weights", T)
    if w13.dtype == torch.float8_e4m3fn:
        _need(w13_scale, torch.float32, "w13_scale", E * 2 * I)
        _need(w2_scale, torch.float32, "w2_scale", E * H)
    if fp4:
        _need(w13_scale, E8M0, "w13_scale", E * 2 * I * (H // 32))
        _need(w2_scale, E8M0, "w2_scale", E * H * (I // 32))
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=x.device)
    _need(out, out_dtype, "out", T * H)
    p = _ffn_params(T, 1, E, H, I, B, w13.dtype, x.dtype, packed, False, False, x_quantized=x_quantized)
    need = moe_grouped_ffn_workspace_bytes(T, 1, E, H, I, B, w13.dtype, x.dtype, False, False)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("moe_grouped_ffn_top1", lib.moe_grouped_ffn_top1(
        ctypes.byref(p), _ptr(x), _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale),
        _ptr(sorted_token_ids), _ptr(expert_ids), _ptr(num_tokens_post_padded), _ptr(topk_ids),
        _ptr(topk_weights), _DT[out_dtype], _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


# ------------------------------------------------------------------ combine --
def moe_combine(y_slots, topk_weights, topk_ids, E, *, out_dtype=torch.bfloat16, out=None,
                stream=None):
    """out[t] = sum_k w[t,k] * y_slots[t*K+k] (ascending k, ids outside [0,E) skipped);
    y_slots fp32, or bf16 (widened exactly to fp32; moe_combine_slots)."""
    lib = load_library()
    T, K = topk_ids.shape
    H = y_slots.shape[1]
    if y_slots.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("y_slots must be float32 or bfloat16")
    _need(y_slots, y_slots.dtype, "y_slots", T * K * H)
    _need(topk_weights, torch.float32, "topk_weights", T * K)
    _need(topk_ids, torch.int32, "topk_ids", T * K)
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=y_slots.device)
    _need(out, out_dtype, "out", T * H)
    if y_slots.dtype == torch.float32:
        _check("moe_combine", lib.moe_combine(T, K, E, H, _ptr(y_slots), _ptr(topk_weights),
                                              _ptr(topk_ids), _DT[out_dtype], _ptr(out),
                                              _stream(stream)))
    else:
        _check("moe_combine_slots", lib.moe_combine_slots(
            T, K, E, H, _ptr(y_slots), _DT[torch.bfloat16], _ptr(topk_weights), _ptr(topk_ids),
            _DT[out_dtype], _ptr(out), _stream(stream)))
    return out


# ------------------------------------------------------- permute/unpermute --
def moe_permute_rows(x, topk_ids, sorted_token_ids, num_tokens_post_padded, E, B, *, x_scale=None,
                     x_perm=None, x_perm_scale=None, row_of_slot=None, stream=None):
    """Rows of x [T, ...] moved into the padded expert order of moe_align_sort:
    returns (x_perm [C, ...], row_of_slot int32 [T*K], x_perm_scale or None).
    Rows of x_perm from num_tokens_post_padded on are not written."""
    lib = load_library()
    T, K = topk_ids.shape
    _need(topk_ids, torch.int32, "topk_ids")
    _need(x, x.dtype, "x")
    if x.shape[0] != T:
        raise ValueError("x and topk_ids disagree on the token count")
    C = moe_align_sort_capacity(T, K, E, B)
    _need(sorted_token_ids, torch.int32, "sorted_token_ids", C)
    _need(num_tokens_post_padded, torch.int32, "num_tokens_post_padded", 1)
    row_bytes = x[0].numel() * x.element_size() if T > 0 else 16
    if x_perm is None:
        x_perm = torch.empty((C,) + tuple(x.shape[1:]), dtype=x.dtype, device=x.device)
    _need(x_perm, x.dtype, "x_perm", C * x[0].numel() if T > 0 else None)
    if row_of_slot is None:
        row_of_slot = torch.empty(T * K, dtype=torch.int32, device=x.device)
    _need(row_of_slot, torch.int32, "row_of_slot", T * K)
    if x_scale is not None:
        _need(x_scale, torch.float32, "x_scale", T)
        if x_perm_scale is None:
            x_perm_scale = torch.empty(C, dtype=torch.float32, device=x.device)
        _need(x_perm_scale, torch.float32, "x_perm_scale", C)
    _check("moe_permute_rows", lib.moe_permute_rows(
        _ptr(x), T, K, E, B, row_bytes, _ptr(topk_ids), _ptr(sorted_token_ids),
        _ptr(num_tokens_post_padded), _ptr(x_scale),
        _ptr(x_perm), _ptr(x_perm_scale if x_scale is not None else None), _ptr(row_of_slot),
        _stream(stream)))
    return x_perm, row_of_slot, (x_perm_scale if x_scale is not None else None)


def moe_unpermute_combine(y_perm, topk_weights, row_of_slot, *, out_dtype=torch.bfloat16, out=None,
                          stream=None, T=None, K=None):
    """out[t] = sum_k w[t,k] * y_perm[row_of_slot[t*K+k]] (ascending k, rows < 0 skipped).
    topk_weights None: every weight is 1 (the gradient of moe_permute_rows);
    then T and K must be given."""
    lib = load_library()
    if topk_weights is not None:
        T, K = topk_weights.shape
        _need(topk_weights, torch.float32, "topk_weights", T * K)
    elif T is None or K is None:
        raise ValueError("unit weights need T and K")
    H = y_perm.shape[1]
    _need(y_perm, torch.float32, "y_perm")
    _need(row_of_slot, torch.int32, "row_of_slot", T * K)
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=y_perm.device)
    _need(out, out_dtype, "out", T * H)
    _check("moe_unpermute_combine", lib.moe_unpermute_combine(
        T, K, H, _ptr(y_perm), _ptr(topk_weights), _ptr(row_of_slot), _DT[out_dtype], _ptr(out),
        _stream(stream)))
    return out


def moe_unpermute_combine_backward(d_out, y_perm, topk_weights, topk_ids, sorted_token_ids,
                                   num_tokens_post_padded, E, B, *, d_y_perm_dtype=torch.float32,
                                   d_y_perm=None, d_topk_weights=None, stream=None):
    """Gradient of moe_unpermute_combine for the upstream d_out [T,H]: returns
    (d_y_perm [C,H], d_topk_weights fp32 [T,K]).  d_y_perm[r] = w[s] d_out[s//K]
    for the slot s in row r < P, zeros for a padding row; rows from P on are
    not written.  d_topk_weights[s] = <d_out[s//K], y_perm[r]>, 0 for a skipped slot."""
    lib = load_library()
    T, K = topk_ids.shape
    H = d_out.shape[1]
    C = moe_align_sort_capacity(T, K, E, B)
    _need(d_out, torch.float32, "d_out", T * H)
    _need(y_perm, torch.float32, "y_perm", C * H)
    _need(topk_weights, torch.float32, "topk_weights", T * K)
    _need(topk_ids, torch.int32, "topk_ids", T * K)
    _need(sorted_token_ids, torch.int32, "sorted_token_ids", C)
    _need(num_tokens_post_padded, torch.int32, "num_tokens_post_padded", 1)
    if d_y_perm is None:
        d_y_perm = torch.empty((C, H), dtype=d_y_perm_dtype, device=d_out.device)
    _need(d_y_perm, d_y_perm_dtype, "d_y_perm", C * H)
    if d_topk_weights is None:
        d_topk_weights = torch.empty((T, K), dtype=torch.float32, device=d_out.device)
    _need(d_topk_weights, torch.float32, "d_topk_weights", T * K)
    _check("moe_unpermute_combine_backward", lib.moe_unpermute_combine_backward(
        T, K, E, B, H, _ptr(d_out), _ptr(y_perm), _ptr(topk_weights), _ptr(topk_ids),
        _ptr(sorted_token_ids), _ptr(num_tokens_post_padded), _DT[d_y_perm_dtype], _ptr(d_y_perm),
        _ptr(d_topk_weights), _stream(stream)))
    return d_y_perm, d_topk_weights


# ---------------------------------------------------------------- backward --
def moe_ffn_backward_workspace_bytes(T, K, E, H, I, B) -> int:
    p = _ffn_params(T, K, E, H, I, B, torch.bfloat16, torch.bfloat16)
    c = int(load_library().moe_ffn_backward_workspace_bytes(ctypes.byref(p)))
    if c < 0:
        raise MoEError("moe_ffn_backward_workspace_bytes", MOE_ERR_UNSUPPORTED)
    return c


def moe_grouped_ffn_train(x, w13, w2, sorted_token_ids, expert_ids, num_tokens_post_padded, *, K, B,
                          y_slots=None, gate_up=None, workspace=None, stream=None, packed=False):
    """moe_grouped_ffn (bf16 weights, canonical or packed) that also keeps the
    fp32 gate and up values of every sorted row for the backward: returns
    (y_slots [T*K,H], gate_up [C,2I])."""
    lib = load_library()
    T, H = x.shape
    E, I, H2 = weight_dims(w13)
    if H2 != H or tuple(w2.shape) != (E, H, I):
        raise ValueError("weight shapes do not match x")
    for t, n in ((x, "x"), (w13, "w13"), (w2, "w2")):
        _need(t, torch.bfloat16, n)
    for t, n in ((sorted_token_ids, "sorted_token_ids"), (expert_ids, "expert_ids"),
                 (num_tokens_post_padded, "num_tokens_post_padded")):
        _need(t, torch.int32, n)
    C = moe_align_sort_capacity(T, K, E, B)
    if y_slots is None:
        y_slots = torch.empty((T * K, H), dtype=torch.float32, device=x.device)
    _need(y_slots, torch.float32, "y_slots", T * K * H)
    if gate_up is None:
        gate_up = torch.empty((C, 2 * I), dtype=torch.float32, device=x.device)
    _need(gate_up, torch.float32, "gate_up", C * 2 * I)
    p = _ffn_params(T, K, E, H, I, B, torch.bfloat16, torch.bfloat16, packed)
    need = moe_grouped_ffn_workspace_bytes(T, K, E, H, I, B, torch.bfloat16, torch.bfloat16)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("moe_grouped_ffn_train", lib.moe_grouped_ffn_train(
        ctypes.byref(p), _ptr(x), _ptr(w13), _ptr(w2), _ptr(sorted_token_ids), _ptr(expert_ids),
        _ptr(num_tokens_post_padded), _ptr(y_slots), _ptr(gate_up), _ptr(workspace), ws_bytes, _stream(stream)))
    return y_slots, gate_up


def moe_ffn_backward(x, w13, w2, topk_ids, topk_weights, sorted_token_ids, expert_ids,
                     num_tokens_post_padded, expert_offsets, y_slots, d_out, *, B, gate_up=None,
                     workspace=None, stream=None, grad_dtype=torch.float32):
    """Gradients of moe_combine(moe_grouped_ffn(...)) for the upstream d_out [T,H]
    (bf16 weights, canonical layout): returns (dx, dw13, dw2, d_topk_weights),
    fp32 except dw13 and dw2 in grad_dtype (fp32 or bf16).
    gate_up: the training forward's gate and up values (else recomputed)."""
    lib = load_library()
    T, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    K = topk_ids.shape[1]
    for t, n, dt in ((x, "x", torch.bfloat16), (w13, "w13", torch.bfloat16), (w2, "w2", torch.bfloat16),
                     (topk_ids, "topk_ids", torch.int32), (topk_weights, "topk_weights", torch.float32),
                     (sorted_token_ids, "sorted_token_ids", torch.int32), (expert_ids, "expert_ids", torch.int32),
                     (num_tokens_post_padded, "num_tokens_post_padded", torch.int32),
                     (expert_offsets, "expert_offsets", torch.int32), (y_slots, "y_slots", torch.float32),
                     (d_out, "d_out", torch.float32)):
        _need(t, dt, n)
    if gate_up is not None:
        _need(gate_up, torch.float32, "gate_up", sorted_token_ids.numel() * I2)
    dev = x.device
    dx = torch.empty((T, H), dtype=torch.float32, device=dev)
    if grad_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("grad_dtype must be float32 or bfloat16")
    dw13 = torch.empty((E, I2, H), dtype=grad_dtype, device=dev)
    dw2 = torch.empty((E, H, I), dtype=grad_dtype, device=dev)
    dwk = torch.empty((T, K), dtype=torch.float32, device=dev)
    p = _ffn_params(T, K, E, H, I, B, torch.bfloat16, torch.bfloat16, grad_dtype=grad_dtype)
    need = moe_ffn_backward_workspace_bytes(T, K, E, H, I, B)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("moe_ffn_backward", lib.moe_ffn_backward(
        ctypes.byref(p), _ptr(x), _ptr(w13), _ptr(w2), _ptr(topk_ids), _ptr(topk_weights),
        _ptr(sorted_token_ids), _ptr(expert_ids), _ptr(num_tokens_post_padded), _ptr(expert_offsets),
        _ptr(y_slots), _ptr(gate_up), _ptr(d_out), _ptr(dx), _ptr(dw13), _ptr(dw2), _ptr(dwk), _ptr(workspace),
        ws_bytes, _stream(stream)))
    return dx, dw13, dw2, dwk


def moe_route_backward(logits, topk_ids, d_topk_weights, K, *, score="softmax", renormalize=True,
                       routed_scaling=1.0, append_shared=False, d_logits=None, stream=None):
    """d_logits [T,E] fp32 for the gradient of the routed columns' weights (selection fixed)."""
    lib = load_library()
    T, E = logits.shape
    _need(logits, torch.float32, "logits")
    _need(topk_ids, torch.int32, "topk_ids")
    _need(d_topk_weights, torch.float32, "d_topk_weights", topk_ids.numel())
    if d_logits is None:
        d_logits = torch.empty((T, E), dtype=torch.float32, device=logits.device)
    _need(d_logits, torch.float32, "d_logits", T * E)
    p = _RouteParams(T, E, K, {"softmax": 0, "sigmoid": 1}[score], 1, 1, int(bool(renormalize)),
                     float(routed_scaling), int(bool(append_shared)))
    _check("moe_route_backward", lib.moe_route_backward(ctypes.byref(p), _ptr(logits), _ptr(topk_ids),
                                                        _ptr(d_topk_weights), _ptr(d_logits),
                                                        _stream(stream)))
    return d_logits


# -------------------------------------------------------------- the layer --
class MoELayer:
    """The four calls of one MoE layer over preallocated buffers.

    Holds the weights and every intermediate buffer so that ``forward`` only
    enqueues the four library calls (route -> align -> grouped FFN -> combine).
    With rows="sorted" the token rows are first moved into the sorted order
    (permute), the FFN reads and writes that order, and the combine reads back
    through the inverse map (route -> align -> permute -> FFN -> unpermute).
    top1: with one slot per token (K 1, no shared expert, rows by token, the
    two-launch schedule, not fp32) "auto" runs the FFN and the combine as one
    call (moe_grouped_ffn_top1; the same output bits); False keeps them apart.
    train: the forward keeps the gate/up values (moe_grouped_ffn_train) and the
    backward reads them instead of recomputing.  grad_dtype: the weight
    gradients' type (float32, or bfloat16: rounded once, half the bytes).
    slot_dtype: the type of the slot rows between the FFN and the combine
    (float32, or bfloat16: half the bytes written and read back; rows by
    token, not fp32 weights, no backward).
    """

    def __init__(self, w13, w2, *, T, K, B, score="softmax", n_group=1, topk_group=1,
                 renormalize=True, routed_scaling=1.0, shared=False, w13_scale=None,
                 w2_scale=None, x_dtype=torch.bfloat16, out_dtype=torch.bfloat16, packed=None,
                 rows="by_token", schedule="two_launch", top1="auto", train=False,
                 grad_dtype=torch.float32, slot_dtype=torch.float32, route_quant="auto"):
        dev = w13.device
        if packed is None:
            packed = w13.dtype != torch.float32
        self.packed = bool(packed)
        E, I, H = weight_dims(w13)
        self.w13_canonical, self.w2_canonical = w13, w2        # what the backward reads
        if self.packed:
            w13, w2 = moe_prepack_weights(w13, w2)
            if w13.dtype == FP4:
                w13_scale, w2_scale = moe_prepack_block_scales(w13_scale, w2_scale, H, I)
        self.w13, self.w2, self.w13_scale, self.w2_scale = w13, w2, w13_scale, w2_scale
        self.E_slabs = E
        self.E_routed = self.E_slabs - (1 if shared else 0)
        self.T, self.K, self.B, self.shared = T, K, B, shared
        self.KO = K + (1 if shared else 0)
        self.H, self.I = H, I
        self.route_kw = dict(score=score, n_group=n_group, topk_group=topk_group,
                             renormalize=renormalize, routed_scaling=routed_scaling,
                             append_shared=shared)
        self.out_dtype = out_dtype
        C = moe_align_sort_capacity(T, self.KO, self.E_slabs, B)
        self.C = C
        self.topk_ids = torch.empty((T, self.KO), dtype=torch.int32, device=dev)
        self.topk_weights = torch.empty((T, self.KO), dtype=torch.float32, device=dev)
        self.sorted = torch.empty(C, dtype=torch.int32, device=dev)
        self.expert_ids = torch.empty(C // B, dtype=torch.int32, device=dev)
        self.ntpp = torch.empty(1, dtype=torch.int32, device=dev)
        self.offsets = torch.empty(self.E_slabs + 1, dtype=torch.int32, device=dev)
        if rows not in ("by_token", "sorted"):
            raise ValueError("rows must be 'by_token' or 'sorted'")
        self.rows_sorted = rows == "sorted"
        if schedule not in ("two_launch", "fused"):
            raise ValueError("schedule must be 'two_launch' or 'fused'")
        self.fused = schedule == "fused"
        ws_a = moe_align_sort_workspace_bytes(T, self.KO, self.E_slabs, B)
        ws_f = moe_grouped_ffn_workspace_bytes(T, self.KO, self.E_slabs, self.H, self.I, B,
                                               w13.dtype, x_dtype, self.rows_sorted, self.fused)
        # where the one-stage schedule reports a wait that gave up (int32, 0 = fine)
        self.status_offset = moe_grouped_ffn_workspace_bytes(
            T, self.KO, self.E_slabs, self.H, self.I, B, w13.dtype, x_dtype, self.rows_sorted) + 32
        self.ws_align = torch.zeros(max(ws_a, 1), dtype=torch.uint8, device=dev)   # zero before first use
        self.ws_ffn = torch.empty(max(ws_f, 1), dtype=torch.uint8, device=dev)
        ny = C if self.rows_sorted else T * self.KO
        if slot_dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("slot_dtype must be float32 or bfloat16")
        if slot_dtype == torch.bfloat16 and (self.rows_sorted or w13.dtype == torch.float32 or train):
            raise ValueError("bf16 slot rows need rows by token, matrix-core weights and no training")
        self.slot_dtype = slot_dtype
        self.y_slots = torch.empty((ny, self.H), dtype=slot_dtype, device=dev)
        if self.rows_sorted:
            self.x_perm = torch.empty((C, self.H), dtype=x_dtype, device=dev)
            self.row_of_slot = torch.empty(T * self.KO, dtype=torch.int32, device=dev)
        self.out = torch.empty((T, self.H), dtype=out_dtype, device=dev)
        eligible = (self.KO == 1 and not self.rows_sorted and not self.fused and w13.dtype != torch.float32)
        if top1 not in ("auto", True, False):
            raise ValueError("top1 must be 'auto', True or False")
        if top1 is True and not eligible:
            raise ValueError("top1 needs K 1 without a shared expert, rows by token, two launches, not fp32")
        self.top1 = eligible and top1 is not False and not train
        self._y_current = False     # y_slots holds the last forward's rows (the backward reads them)
        # train: the forward also keeps the gate/up values, and the backward reads them
        self.train = bool(train)
        self.grad_dtype = grad_dtype
        self.gate_up = None
        if self.train:
            if w13.dtype != torch.bfloat16 or self.rows_sorted or self.fused:
                raise ValueError("train needs bf16 weights, rows by token and two launches")
            self.gate_up = torch.empty((C, 2 * I), dtype=torch.float32, device=dev)
        self._gu_current = False
        # E4M3 / MXFP4 weights with token rows: the forward routes and
        # quantises the activations in one launch (moe_route_topk_quantize)
        quant_ok = w13.dtype in (torch.float8_e4m3fn, FP4) and not self.rows_sorted and x_dtype == torch.bfloat16
        if route_quant not in ("auto", True, False):
            raise ValueError("route_quant must be 'auto', True or False")
        if route_quant is True and not quant_ok:
            raise ValueError("route_quant needs E4M3 or MXFP4 weights, bf16 x and rows by token")
        self.route_quant = quant_ok and route_quant is not False
        self.w_dtype = w13.dtype

    def route(self, logits, bias=None):
        return moe_route_topk(logits, self.K, bias=bias, topk_ids=self.topk_ids,
                              topk_weights=self.topk_weights, **self.route_kw)

    def route_quantize(self, x, logits, bias=None):
        """Routing and the activation quantisation of x into the FFN workspace, one launch."""
        return moe_route_topk_quantize(logits, self.K, x, self.ws_ffn, w13=self.w13, B=self.B, K_ffn=self.KO,
                                       bias=bias, fused=self.fused, topk_ids=self.topk_ids,
                                       topk_weights=self.topk_weights, **self.route_kw)

    def align(self):
        return moe_align_sort(self.topk_ids, self.E_slabs, self.B, sorted_token_ids=self.sorted,
                              expert_ids=self.expert_ids, num_tokens_post_padded=self.ntpp,
                              expert_offsets=self.offsets, workspace=self.ws_align)

    def permute(self, x):
        return moe_permute_rows(x, self.topk_ids, self.sorted, self.ntpp, self.E_slabs, self.B,
                                x_perm=self.x_perm, row_of_slot=self.row_of_slot)

    def ffn(self, x, stage_events=None, x_quantized=False):
        self._y_current = True
        self._gu_current = False
        if self.rows_sorted:
            return moe_grouped_ffn(self.x_perm, self.w13, self.w2, self.sorted, self.expert_ids,
                                   self.ntpp, K=self.KO, B=self.B, w13_scale=self.w13_scale,
                                   w2_scale=self.w2_scale, y_slots=self.y_slots,
                                   workspace=self.ws_ffn, stage_events=stage_events,
                                   packed=self.packed, T=self.T, fused=self.fused)
        return moe_grouped_ffn(x, self.w13, self.w2, self.sorted, self.expert_ids, self.ntpp,
                               K=self.KO, B=self.B, w13_scale=self.w13_scale,
                               w2_scale=self.w2_scale, y_slots=self.y_slots, workspace=self.ws_ffn,
                               stage_events=stage_events, packed=self.packed, fused=self.fused,
                               x_quantized=x_quantized)

    def fused_status(self):
        """The one-stage schedule's status word (0 = every wait was satisfied); syncs."""
        if not self.fused:
            return 0
        return int(self.ws_ffn[self.status_offset:self.status_offset + 4].view(torch.int32).item())

    def combine(self):
        if self.rows_sorted:
            return moe_unpermute_combine(self.y_slots, self.topk_weights, self.row_of_slot,
                                         out_dtype=self.out_dtype, out=self.out)
        return moe_combine(self.y_slots, self.topk_weights, self.topk_ids, self.E_slabs,
                           out_dtype=self.out_dtype, out=self.out)

    def ffn_train(self, x):
        """The training forward's FFN: slot rows plus the gate/up values the backward reads."""
        self._y_current = True
        self._gu_current = True
        return moe_grouped_ffn_train(x, self.w13, self.w2, self.sorted, self.expert_ids, self.ntpp, K=self.KO,
                                     B=self.B, y_slots=self.y_slots, gate_up=self.gate_up,
                                     workspace=self.ws_ffn, packed=self.packed)

    def ffn_top1(self, x, x_quantized=False):
        """The FFN and the combine of a top-1 layer in one call (into self.out)."""
        self._y_current = False
        self._gu_current = False
        return moe_grouped_ffn_top1(x, self.w13, self.w2, self.sorted, self.expert_ids, self.ntpp,
                                    self.topk_ids, self.topk_weights, B=self.B, w13_scale=self.w13_scale,
                                    w2_scale=self.w2_scale, out_dtype=self.out_dtype, out=self.out,
                                    workspace=self.ws_ffn, packed=self.packed, x_quantized=x_quantized)

    def backward(self, x, logits, d_out, workspace=None, recompute=False):
        """Gradients after forward(x, logits): (dx, dw13, dw2, d_logits), fp32.
        The backward reads the forward's slot rows; after a top-1 forward,
        which does not write them, they are recomputed first.  After a training
        forward it reads the kept gate/up values unless recompute is set."""
        if self.slot_dtype != torch.float32:
            raise ValueError("the backward reads fp32 slot rows: build the layer with slot_dtype float32")
        if not self._y_current:
            self.ffn(x)
        dx, dw13, dw2, dwk = moe_ffn_backward(
            x, self.w13_canonical, self.w2_canonical, self.topk_ids, self.topk_weights, self.sorted,
            self.expert_ids, self.ntpp, self.offsets, self.y_slots, d_out, B=self.B,
            gate_up=self.gate_up if (self._gu_current and not recompute) else None, workspace=workspace,
            grad_dtype=self.grad_dtype)
        d_logits = moe_route_backward(logits, self.topk_ids, dwk, self.K, score=self.route_kw["score"],
                                      renormalize=self.route_kw["renormalize"],
                                      routed_scaling=self.route_kw["routed_scaling"],
                                      append_shared=self.shared)
        return dx, dw13, dw2, d_logits, dwk

    def forward(self, x, logits, bias=None):
        if self.route_quant:
            self.route_quantize(x, logits, bias)
        else:
            self.route(logits, bias)
        self.align()
        if self.rows_sorted:
            self.permute(x)
        if self.top1:
            return self.ffn_top1(x, x_quantized=self.route_quant)
        if self.train:
            self.ffn_train(x)
        else:
            self.ffn(x, x_quantized=self.route_quant)
        return self.combine()


# ------------------------------------------------------------ HIP events --
class HipEvents:
    """A pool of timing hipEvent_t handles (for measuring stages on a stream).

    Created with hipEventDisableSystemFence: they only time work, so recording
    them skips the system-scope cache writeback an ordinary event adds between
    kernels (read them after synchronising the stream)."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, n):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self._hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                  ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.handles = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self._hip.hipEventCreateWithFlags(ctypes.byref(h), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.handles.append(h.value)

    def record(self, i, stream=None):
        if self._hip.hipEventRecord(ctypes.c_void_p(self.handles[i]), _stream(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, i, j):
        ms = ctypes.c_float()
        st = self._hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.handles[i]),
                                           ctypes.c_void_p(self.handles[j]))
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return float(ms.value)

    def close(self):
        for h in self.handles:
            self._hip.hipEventDestroy(ctypes.c_void_p(h))
        self.handles = []
