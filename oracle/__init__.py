"""CPU oracle for the single-GPU MoE FFN layer.

TEST INFRASTRUCTURE ONLY.  The test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only code allowed to import this
package.  The product library (``routing_align_sort_amd``) never imports it and
shares no code with it: the arithmetic lives in ``moe_oracle.c`` (plain C,
double precision), which this module compiles with gcc and calls through
ctypes.  Everything here is argument marshalling between numpy arrays and that
C code.

Each function names the passage of the pages it follows in ``moe_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None

SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1
W_F32, W_BF16, W_E4M3, W_MXFP4 = 0, 1, 2, 3
X_F32, X_BF16 = 0, 1
INTER_F64, INTER_F32, INTER_BF16, INTER_E4M3 = 0, 1, 2, 3


def build(force: bool = True) -> str:
    """Compile moe_oracle.c into libmoe_oracle.so (gcc, OpenMP, no FMA contraction)."""
    global _lib
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_bf16_encode_array.argtypes = [P, i64, P]
    lib.oracle_bf16_decode_array.argtypes = [P, i64, P]
    lib.oracle_e4m3_encode_array.argtypes = [P, i64, P]
    lib.oracle_e4m3_decode_array.argtypes = [P, i64, P]
    lib.oracle_e2m1_decode_array.argtypes = [P, i64, P]
    lib.oracle_e8m0_decode_array.argtypes = [P, i64, P]
    for f in (lib.oracle_bf16_encode_array, lib.oracle_bf16_decode_array,
              lib.oracle_e4m3_encode_array, lib.oracle_e4m3_decode_array,
              lib.oracle_e2m1_decode_array, lib.oracle_e8m0_decode_array):
        f.restype = None
    lib.oracle_route_topk.argtypes = [i32, i32, i32, i32, i32, i32, i32, f64, i32, P, P, P, P]
    lib.oracle_route_topk.restype = i32
    lib.oracle_align_capacity.argtypes = [i64, i64, i64]
    lib.oracle_align_capacity.restype = i64
    lib.oracle_align_sort.argtypes = [P, i32, i32, i32, i32, P, P, P, P]
    lib.oracle_align_sort.restype = i32
    lib.oracle_quant_tokens_e4m3.argtypes = [P, i32, i32, P, P]
    lib.oracle_quant_tokens_e4m3.restype = None
    lib.oracle_quant_row_e4m3.argtypes = [P, i64, P, P]
    lib.oracle_quant_row_e4m3.restype = None
    lib.oracle_expert_ffn.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32,
                                      P, P, P, P, P, P, P]
    lib.oracle_expert_ffn.restype = i32
    lib.oracle_combine.argtypes = [i32, i32, i32, i32, P, P, P, P]
    lib.oracle_combine.restype = i32
    lib.oracle_permute_rows.argtypes = [P, i32, i64, i32, P, i64, P]
    lib.oracle_permute_rows.restype = i32
    lib.oracle_row_of_slot.argtypes = [P, i64, i64, P]
    lib.oracle_row_of_slot.restype = i32
    lib.oracle_unpermute_combine.argtypes = [i32, i32, i32, P, P, P, P]
    lib.oracle_unpermute_combine.restype = i32
    lib.oracle_unpermute_combine_backward.argtypes = [i32, i32, i32, P, P, P, P, i64, i32, P, P]
    lib.oracle_unpermute_combine_backward.restype = i32
    lib.oracle_ffn_backward.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P,
                                        P, P, P, P]
    lib.oracle_ffn_backward.restype = i32
    lib.oracle_route_backward.argtypes = [i32, i32, i32, i32, i32, f64, i32, P, P, P, P]
    lib.oracle_route_backward.restype = i32
    lib.oracle_num_threads.restype = i32
    lib.oracle_set_num_threads.argtypes = [i32]
    lib.oracle_set_num_threads.restype = None
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def set_num_threads(n: int) -> None:
    """Threads of the oracle's OpenMP loops (for timing it on one core)."""
    _load().oracle_set_num_threads(int(n))


def num_threads() -> int:
    """Threads of the oracle's OpenMP loop over token slots."""
    return int(_load().oracle_num_threads())


# ---------------------------------------------------------------- codecs ----
def bf16_encode(v) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint16)
    _load().oracle_bf16_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def bf16_decode(b) -> np.ndarray:
    b = _c(b, np.uint16)
    out = np.empty(b.shape, np.float64)
    _load().oracle_bf16_decode_array(_ptr(b), b.size, _ptr(out))
    return out


def e4m3_encode(v) -> np.ndarray:
    """fp32 -> OCP E4M3 codes (uint8), nearest even, saturating at +-448."""
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().oracle_e4m3_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def e4m3_decode(c) -> np.ndarray:
    c = _c(c, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().oracle_e4m3_decode_array(_ptr(c), c.size, _ptr(out))
    return out


def e2m1_decode(nibbles) -> np.ndarray:
    """OCP MX FP4 (E2M1) element codes (one per uint8, low 4 bits) -> values."""
    c = _c(nibbles, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().oracle_e2m1_decode_array(_ptr(c), c.size, _ptr(out))
    return out


def e8m0_decode(e) -> np.ndarray:
    """E8M0 block scales (uint8) -> 2^(e-127) (NaN for 255)."""
    c = _c(e, np.uint8)
    out = np.empty(c.shape, np.float64)
    _load().oracle_e8m0_decode_array(_ptr(c), c.size, _ptr(out))
    return out


# --------------------------------------------------------------- routing ----
def route_topk(logits, K, *, score="softmax", bias=None, n_group=1, topk_group=1,
               renormalize=True, routed_scaling=1.0, append_shared=False):
    """Top-K routing of each token (row of ``logits``); returns (ids, weights).

    ids int32 [T, K(+1)], weights float32 [T, K(+1)]; see moe_oracle.c.
    """
    logits = _c(logits, np.float32)
    T, E = logits.shape
    b = None if bias is None else _c(bias, np.float32)
    KO = K + (1 if append_shared else 0)
    ids = np.empty((T, KO), np.int32)
    w = np.empty((T, KO), np.float32)
    mode = {"softmax": SCORE_SOFTMAX, "sigmoid": SCORE_SIGMOID}[score]
    rc = _load().oracle_route_topk(T, E, K, mode, n_group, topk_group, int(bool(renormalize)),
                                   float(routed_scaling), int(bool(append_shared)),
                                   _ptr(logits), _ptr(b), _ptr(ids), _ptr(w))
    if rc != 0:
        raise ValueError("oracle_route_topk: invalid arguments")
    return ids, w


# ----------------------------------------------------------- align&sort ----
def align_capacity(S: int, E: int, B: int) -> int:
    return int(_load().oracle_align_capacity(S, E, B))


def align_sort(topk_ids, E: int, B: int):
    """Stable counting sort of the token slots by expert with per-expert padding.

    Returns dict(sorted_token_ids [C], expert_ids [C/B], num_tokens_post_padded,
    expert_offsets [E+1]).
    """
    ids = _c(topk_ids, np.int32)
    if ids.ndim == 1:
        ids = ids.reshape(-1, 1)
    T, K = ids.shape
    C = align_capacity(T * K, E, B)
    sorted_ids = np.empty(C, np.int32)
    expert_ids = np.empty(C // B, np.int32)
    P = np.zeros(1, np.int32)
    off = np.empty(E + 1, np.int32)
    rc = _load().oracle_align_sort(_ptr(ids), T, K, E, B, _ptr(sorted_ids), _ptr(expert_ids),
                                   _ptr(P), _ptr(off))
    if rc != 0:
        raise ValueError("oracle_align_sort: invalid arguments")
    return {"sorted_token_ids": sorted_ids, "expert_ids": expert_ids,
            "num_tokens_post_padded": int(P[0]), "expert_offsets": off}


# ----------------------------------------------------------- fp8 quant ----
def quant_tokens_e4m3(x_bf16):
    """Per-token E4M3 quantisation of bf16 rows; returns (codes uint8, scales f32)."""
    x = _c(x_bf16, np.uint16)
    T, H = x.shape
    q = np.empty((T, H), np.uint8)
    s = np.empty(T, np.float32)
    _load().oracle_quant_tokens_e4m3(_ptr(x), T, H, _ptr(q), _ptr(s))
    return q, s


def quant_row_e4m3(v):
    """E4M3 quantisation of one fp32 row with a per-row scale; returns (codes, scale)."""
    v = _c(v, np.float32).ravel()
    q = np.empty(v.size, np.uint8)
    s = np.empty(1, np.float32)
    _load().oracle_quant_row_e4m3(_ptr(v), v.size, _ptr(q), _ptr(s))
    return q, float(s[0])


# ------------------------------------------------------------ FFN, combine ----
_WDT = {"f32": (W_F32, np.float32), "bf16": (W_BF16, np.uint16), "e4m3": (W_E4M3, np.uint8),
        "e2m1": (W_MXFP4, np.uint8)}
_XDT = {"f32": (X_F32, np.float32), "bf16": (X_BF16, np.uint16)}
_INTER = {"f64": INTER_F64, "f32": INTER_F32, "bf16": INTER_BF16, "e4m3": INTER_E4M3}


def expert_ffn(x, w13, w2, topk_ids, *, w_dtype, x_dtype, inter, w13_scale=None, w2_scale=None):
    """y_slots[t*K+k] = FFN_{ids[t,k]}(x[t]) as float32 [T*K, H].

    x: [T,H] fp32 or bf16 bit patterns; w13 [E,2I,H], w2 [E,H,I] in fp32, bf16 bits
    or E4M3 codes (with fp32 w13_scale [E,2I], w2_scale [E,H]); for "e2m1"
    (MXFP4) w13 [E,2I,H/2], w2 [E,H,I/2] bytes of two codes each, with E8M0
    block scales w13_scale [E,2I,H/32], w2_scale [E,H,I/32] (uint8).  Slots
    with ids out of range are left at zero.
    """
    wcode, wnp = _WDT[w_dtype]
    xcode, xnp = _XDT[x_dtype]
    x = _c(x, xnp)
    w13 = _c(w13, wnp)
    w2 = _c(w2, wnp)
    ids = _c(topk_ids, np.int32)
    T, H = x.shape
    K = ids.shape[1]
    E, I2, H2 = w13.shape
    I = I2 // 2
    fp4 = w_dtype == "e2m1"
    if fp4:
        assert H2 * 2 == H and w2.shape == (E, H, I // 2) and ids.shape[0] == T
    else:
        assert H2 == H and w2.shape == (E, H, I) and ids.shape[0] == T
    snp = np.uint8 if fp4 else np.float32
    s13 = None if w13_scale is None else _c(w13_scale, snp)
    s2 = None if w2_scale is None else _c(w2_scale, snp)
    if fp4 and s13 is not None:
        assert s13.shape == (E, 2 * I, H // 32) and s2.shape == (E, H, I // 32)
    y = np.zeros((T * K, H), np.float32)
    rc = _load().oracle_expert_ffn(T, K, E, H, I, wcode, xcode, _INTER[inter], _ptr(x), _ptr(w13),
                                   _ptr(s13), _ptr(w2), _ptr(s2), _ptr(ids), _ptr(y))
    if rc != 0:
        raise ValueError("oracle_expert_ffn: invalid arguments")
    return y


def combine(y_slots, topk_weights, topk_ids, E: int):
    """out[t] = sum_k w[t,k] * y_slots[t*K+k] (double, ascending k, ids out of range skipped)."""
    y = _c(y_slots, np.float32)
    w = _c(topk_weights, np.float32)
    ids = _c(topk_ids, np.int32)
    T, K = ids.shape
    H = y.shape[1]
    out = np.empty((T, H), np.float64)
    rc = _load().oracle_combine(T, K, E, H, _ptr(y), _ptr(w), _ptr(ids), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_combine: invalid arguments")
    return out


def moe_layer(x, w13, w2, topk_ids, topk_weights, *, w_dtype, x_dtype, inter,
              w13_scale=None, w2_scale=None, E=None):
    """The expert FFN of every slot followed by the combine: (out f64 [T,H], y_slots)."""
    E = w13.shape[0] if E is None else E
    y = expert_ffn(x, w13, w2, topk_ids, w_dtype=w_dtype, x_dtype=x_dtype, inter=inter,
                   w13_scale=w13_scale, w2_scale=w2_scale)
    return combine(y, topk_weights, topk_ids, E), y


def permute_rows(x, sorted_ids, K: int, P=None, out=None):
    """Rows of x (any dtype, [T, ...]) moved into the padded expert order: for
    r < P (default: every row of sorted_ids), row r is x[sorted_ids[r] // K]
    where sorted_ids[r] < T*K, else zeros; rows from P on keep the contents of
    ``out`` (zeros when not given)."""
    xa = np.ascontiguousarray(x)
    T = xa.shape[0]
    row_bytes = xa.dtype.itemsize * (int(np.prod(xa.shape[1:])) if xa.ndim > 1 else 1)
    srt = _c(sorted_ids, np.int32)
    C = srt.shape[0]
    P = C if P is None else int(P)
    if out is None:
        out = np.zeros((C,) + xa.shape[1:], xa.dtype)
    else:
        out = np.array(out, dtype=xa.dtype, copy=True).reshape((C,) + xa.shape[1:])
    rc = _load().oracle_permute_rows(_ptr(xa), T, row_bytes, K, _ptr(srt), P, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_permute_rows: invalid arguments")
    return out


def row_of_slot(sorted_ids, S: int):
    """Inverse of the padded layout: the row holding each slot, -1 if none."""
    srt = _c(sorted_ids, np.int32)
    out = np.empty(S, np.int32)
    rc = _load().oracle_row_of_slot(_ptr(srt), srt.shape[0], S, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_row_of_slot: invalid arguments")
    return out


def unpermute_combine(y_perm, topk_weights, row_of_slot_):
    """out[t] = sum_k w[t,k] * y_perm[row_of_slot[t*K+k]] (double, ascending k, -1 skipped)."""
    y = _c(y_perm, np.float32)
    w = _c(topk_weights, np.float32)
    rs = _c(row_of_slot_, np.int32)
    T, K = w.shape
    H = y.shape[1]
    out = np.empty((T, H), np.float64)
    rc = _load().oracle_unpermute_combine(T, K, H, _ptr(y), _ptr(w), _ptr(rs), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_unpermute_combine: invalid arguments")
    return out


def unpermute_combine_backward(d_out, y_perm, topk_weights, sorted_ids, P=None, round_to="f64"):
    """Gradient of unpermute_combine for an upstream d_out [T,H]: (d_y_perm
    float64 [P,H], d_w float64 [T,K]).  d_y_perm[r] = w[s] d_out[s // K] for
    the slot s in row r, zeros for padding rows; d_w[s] = <d_out[s // K],
    y_perm[row of s]>, 0 for a slot that was not placed.  round_to: "f64"
    (exact), "f32" or "bf16" (fp32 product rounded to bf16), as delivered."""
    g = _c(d_out, np.float32)
    y = _c(y_perm, np.float32)
    w = _c(topk_weights, np.float32)
    srt = _c(sorted_ids, np.int32)
    T, K = w.shape
    H = g.shape[1]
    P = srt.shape[0] if P is None else int(P)
    rnd = {"f64": 0, "f32": 1, "bf16": 2}[round_to]
    dy = np.empty((P, H), np.float64)
    dw = np.empty((T, K), np.float64)
    rc = _load().oracle_unpermute_combine_backward(T, K, H, _ptr(g), _ptr(y), _ptr(w), _ptr(srt), P, rnd,
                                                   _ptr(dy), _ptr(dw))
    if rc != 0:
        raise ValueError("oracle_unpermute_combine_backward: invalid arguments")
    return dy, dw


def ffn_backward(x, w13, w2, topk_ids, topk_weights, y_slots, d_out, *, w_dtype, x_dtype, inter):
    """Gradients of the layer (expert FFNs + combine) for an upstream d_out [T,H]:
    (dx [T,H], dW13 [E,2I,H], dW2 [E,H,I], d_w [T,K]), all float64.
    w_dtype / x_dtype "f32" or "bf16" (bits); inter "f64" (no rounding) or "bf16"."""
    wcode, wnp = _WDT[w_dtype]
    xcode, xnp = _XDT[x_dtype]
    if wcode > 1:
        raise ValueError("the backward covers fp32 and bf16 weights")
    x = _c(x, xnp)
    w13 = _c(w13, wnp)
    w2 = _c(w2, wnp)
    ids = _c(topk_ids, np.int32)
    w = _c(topk_weights, np.float32)
    y = _c(y_slots, np.float32)
    dout = _c(d_out, np.float32)
    T, H = x.shape
    K = ids.shape[1]
    E, I2, _ = w13.shape
    I = I2 // 2
    dx = np.empty((T, H), np.float64)
    dw13 = np.empty((E, I2, H), np.float64)
    dw2 = np.empty((E, H, I), np.float64)
    dwk = np.empty((T, K), np.float64)
    rc = _load().oracle_ffn_backward(T, K, E, H, I, wcode, xcode, _INTER[inter], _ptr(x), _ptr(w13),
                                     _ptr(w2), _ptr(ids), _ptr(w), _ptr(y), _ptr(dout), _ptr(dx),
                                     _ptr(dw13), _ptr(dw2), _ptr(dwk))
    if rc != 0:
        raise ValueError("oracle_ffn_backward: invalid arguments")
    return dx, dw13, dw2, dwk


def route_backward(logits, topk_ids, d_w, K: int, *, score="softmax", renormalize=True,
                   routed_scaling=1.0, append_shared=False):
    """d_logits [T,E] (float64) for d_w over the routed columns, the selection held fixed."""
    lg = _c(logits, np.float32)
    ids = _c(topk_ids, np.int32)
    dw = _c(d_w, np.float32)
    T, E = lg.shape
    out = np.empty((T, E), np.float64)
    rc = _load().oracle_route_backward(T, E, K, {"softmax": 0, "sigmoid": 1}[score], int(bool(renormalize)),
                                       float(routed_scaling), int(bool(append_shared)), _ptr(lg),
                                       _ptr(ids), _ptr(dw), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_route_backward: invalid arguments")
    return out
