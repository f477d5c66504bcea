"""The C-ABI library on a host without a GPU: it loads, exports every function
include/moe_mi355x.h declares, and its host-side validation and sizing work
(none of these calls touches the device)."""
import ctypes
import os
import re

import pytest

import routing_align_sort_amd as moe
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        from routing_align_sort_amd import build
        build.build()
    return moe.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 24, names
    assert set(names) == set(moe.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert moe.abi_version() == 10
    assert moe.status_string(0) == "ok"
    assert "workspace" in moe.status_string(3)
    assert moe.status_string(99) == "unknown status"


def test_capacity_matches_oracle_closed_form(lib):
    for T, K, E, B in [(0, 1, 1, 1), (1, 1, 1, 16), (16384, 8, 256, 64), (64, 8, 256, 16),
                       (2048, 2, 33, 32), (5, 3, 1024, 128), (3, 2, 7, 5)]:
        assert moe.moe_align_sort_capacity(T, K, E, B) == oracle.align_capacity(T * K, E, B)


def test_invalid_arguments_are_rejected_on_the_host(lib):
    P = ctypes.c_void_p
    assert lib.moe_align_sort_capacity(-1, 1, 1, 1) == -1
    assert lib.moe_align_sort_capacity(1, 0, 1, 1) == -1
    assert lib.moe_align_sort_workspace_bytes(1, 1, 0, 1) == -1
    # E beyond the built limit
    st = lib.moe_align_sort(None, 1, 1, 2000, 1, None, None, P(8), None, None, 0, None)
    assert st == moe.MOE_ERR_UNSUPPORTED
    # null output pointer
    st = lib.moe_align_sort(P(8), 4, 2, 8, 16, None, P(8), P(8), None, None, 0, None)
    assert st == moe.MOE_ERR_INVALID_ARG
    # the multi-block path needs a workspace
    need = lib.moe_align_sort_workspace_bytes(16384, 8, 256, 64)
    assert need > 0
    st = lib.moe_align_sort(P(8), 16384, 8, 256, 64, P(8), P(8), P(8), None, None, need - 1, None)
    assert st == moe.MOE_ERR_WORKSPACE
    assert lib.moe_align_sort_workspace_bytes(64, 8, 256, 16) == 0     # one workgroup, no workspace


def test_no_alloc_align_sort_limit_is_checked_on_the_host(lib):
    # beyond the fixed scratch: rejected before the device is touched
    P = ctypes.c_void_p
    limit = lib.moe_align_sort_noalloc_scratch_bytes()
    assert limit == 1088 * 1024
    assert lib.moe_align_sort_workspace_bytes(1 << 20, 8, 1024, 16) > limit
    st = lib.moe_align_sort_noalloc(P(8), 1 << 20, 8, 1024, 16, P(8), P(8), P(8), None, None)
    assert st == moe.MOE_ERR_SCRATCH_LIMIT
    assert "scratch" in moe.status_string(st)
    # the same argument checks as the workspace call
    assert lib.moe_align_sort_noalloc(P(8), 4, 2, 8, 16, None, P(8), P(8), None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_align_sort_noalloc(None, 1, 1, 2000, 1, None, None, P(8), None, None) == moe.MOE_ERR_UNSUPPORTED


def test_route_validation(lib):
    p = moe._RouteParams(4, 256, 8, 1, 8, 4, 1, 1.0, 0)
    P = ctypes.c_void_p
    p.K = 0
    assert lib.moe_route_topk(ctypes.byref(p), P(8), None, P(8), P(8), None) == moe.MOE_ERR_INVALID_ARG
    p.K = 8; p.n_group = 7
    assert lib.moe_route_topk(ctypes.byref(p), P(8), None, P(8), P(8), None) == moe.MOE_ERR_INVALID_ARG
    p.n_group = 8; p.topk_group = 1; p.K = 33                # only 32 experts eligible
    assert lib.moe_route_topk(ctypes.byref(p), P(8), None, P(8), P(8), None) == moe.MOE_ERR_INVALID_ARG
    p.topk_group = 4; p.K = 8; p.E = 2048; p.n_group = 8
    assert lib.moe_route_topk(ctypes.byref(p), P(8), None, P(8), P(8), None) == moe.MOE_ERR_UNSUPPORTED
    p.E = 256; p.T = 0
    assert lib.moe_route_topk(ctypes.byref(p), None, None, None, None, None) == moe.MOE_OK


def test_ffn_validation_and_workspace(lib):
    import torch
    ws = moe.moe_grouped_ffn_workspace_bytes(2048, 1, 32, 7168, 2048, 64, torch.bfloat16, torch.bfloat16)
    C = oracle.align_capacity(2048, 32, 64)
    assert ws >= C * 2048 * 2
    with pytest.raises(moe.MoEError):
        moe.moe_grouped_ffn_workspace_bytes(64, 2, 8, 128, 256, 48, torch.bfloat16, torch.bfloat16)
    with pytest.raises(moe.MoEError):       # H not a multiple of the tile
        moe.moe_grouped_ffn_workspace_bytes(64, 2, 8, 100, 256, 16, torch.bfloat16, torch.bfloat16)
    with pytest.raises(moe.MoEError):       # fp8 activations are not a built combination
        moe.moe_grouped_ffn_workspace_bytes(64, 2, 8, 256, 256, 16, torch.float8_e4m3fn,
                                            torch.float8_e4m3fn)
    p = moe._FfnParams(64, 2, 8, 256, 256, 16, 1, 1, 0)
    P = ctypes.c_void_p
    st = lib.moe_grouped_ffn(ctypes.byref(p), P(8), P(8), None, P(8), None, P(8), P(8), P(8), P(8),
                             P(8), 10, None)
    assert st == moe.MOE_ERR_WORKSPACE
    p.w_dtype = 2
    st = lib.moe_grouped_ffn(ctypes.byref(p), P(8), P(8), None, P(8), None, P(8), P(8), P(8), P(8),
                             P(8), 1 << 30, None)
    assert st == moe.MOE_ERR_INVALID_ARG        # fp8 needs its scales
    p.w_dtype = 1; p.weight_layout = 5
    st = lib.moe_grouped_ffn(ctypes.byref(p), P(8), P(8), None, P(8), None, P(8), P(8), P(8), P(8),
                             P(8), 1 << 30, None)
    assert st == moe.MOE_ERR_INVALID_ARG        # unknown weight layout
    f = moe._FfnParams(64, 2, 8, 256, 256, 16, 0, 0, 1)
    assert lib.moe_prepack_weights(ctypes.byref(f), P(8), P(8), P(16), P(16), None) == moe.MOE_ERR_UNSUPPORTED
    f.w_dtype = 1
    assert lib.moe_prepack_weights(ctypes.byref(f), P(8), P(8), P(8), P(16), None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_combine(4, 2, 8, 6, P(8), P(8), P(8), 1, P(8), None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_combine(4, 2, 8, 8, P(8), P(8), P(8), 7, P(8), None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_combine(0, 2, 8, 8, None, None, None, 1, None, None) == moe.MOE_OK


def test_mxfp4_validation(lib):
    import torch
    P = ctypes.c_void_p
    # E2M1 weights take bf16 activations and the fp8 workspace layout
    ws4 = moe.moe_grouped_ffn_workspace_bytes(64, 8, 256, 7168, 2048, 16, moe.FP4, torch.bfloat16)
    ws8 = moe.moe_grouped_ffn_workspace_bytes(64, 8, 256, 7168, 2048, 16, torch.float8_e4m3fn,
                                              torch.bfloat16)
    assert ws4 == ws8
    p = moe._FfnParams(64, 2, 8, 256, 256, 16, moe.MOE_FP4_E2M1, moe.MOE_BF16, 0)
    st = lib.moe_grouped_ffn(ctypes.byref(p), P(8), P(8), None, P(8), P(8), P(8), P(8), P(8), P(8),
                             P(8), 1 << 30, None)
    assert st == moe.MOE_ERR_INVALID_ARG        # block scales are required
    p.x_dtype = moe.MOE_FP4_E2M1
    assert lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(p)) == -1
    # block-scale packing: only for E2M1, sizes as for the weights, no aliasing
    f = moe._FfnParams(1, 1, 8, 256, 256, 16, moe.MOE_FP8_E4M3, moe.MOE_BF16, 1)
    assert lib.moe_prepack_block_scales(ctypes.byref(f), P(8), P(8), P(16), P(24), None) == \
        moe.MOE_ERR_UNSUPPORTED
    f.w_dtype = moe.MOE_FP4_E2M1; f.I = 192
    assert lib.moe_prepack_block_scales(ctypes.byref(f), P(8), P(8), P(16), P(24), None) == \
        moe.MOE_ERR_UNSUPPORTED
    f.I = 256
    assert lib.moe_prepack_block_scales(ctypes.byref(f), P(8), P(8), P(8), P(24), None) == \
        moe.MOE_ERR_INVALID_ARG
    assert lib.moe_prepack_block_scales(ctypes.byref(f), None, P(8), P(16), P(24), None) == \
        moe.MOE_ERR_INVALID_ARG


def test_activation_operand_limit(lib):
    import torch
    # x of 2^20 tokens x 2048 bf16 = 4 GiB fits; one more token does not
    assert moe.moe_grouped_ffn_workspace_bytes(1 << 20, 1, 8, 2048, 128, 16, torch.bfloat16,
                                               torch.bfloat16) > 0
    with pytest.raises(moe.MoEError):
        moe.moe_grouped_ffn_workspace_bytes((1 << 20) + 1, 1, 8, 2048, 128, 16, torch.bfloat16,
                                            torch.bfloat16)
    # the quantised paths read one byte per element
    assert moe.moe_grouped_ffn_workspace_bytes((1 << 20) + 1, 1, 8, 2048, 128, 16,
                                               torch.float8_e4m3fn, torch.bfloat16) > 0


def test_permute_and_row_layout_validation(lib):
    import torch
    P = ctypes.c_void_p
    # row bytes must be a positive multiple of 16; scales come in pairs
    st = lib.moe_permute_rows(P(8), 4, 2, 8, 16, 24, P(8), P(8), P(8), None, P(8), None, P(8), None)
    assert st == moe.MOE_ERR_INVALID_ARG
    st = lib.moe_permute_rows(P(8), 4, 2, 8, 16, 32, P(8), P(8), P(8), P(8), P(8), None, P(8), None)
    assert st == moe.MOE_ERR_INVALID_ARG
    st = lib.moe_permute_rows(P(8), 4, 2, 8, 16, 32, P(8), P(8), P(8), None, P(8), None, None, None)
    assert st == moe.MOE_ERR_INVALID_ARG       # the inverse map is required
    st = lib.moe_permute_rows(P(8), 4, 2, 8, 16, 32, P(8), P(8), None, None, P(8), None, P(8), None)
    assert st == moe.MOE_ERR_INVALID_ARG       # and the padded row count
    assert lib.moe_permute_rows(None, 0, 2, 8, 16, 32, None, None, None, None, None, None, None,
                                None) == moe.MOE_OK
    assert lib.moe_unpermute_combine(4, 2, 6, P(8), P(8), P(8), 1, P(8), None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_unpermute_combine(4, 2, 8, None, P(8), P(8), 1, P(8), None) == moe.MOE_ERR_INVALID_ARG
    # the top-1 FFN + combine: K must be 1; fp32, sorted rows and the one-stage schedule are not built
    t1 = lib.moe_grouped_ffn_top1
    q = moe._FfnParams(64, 1, 8, 256, 256, 16, 1, 1, 0, moe.MOE_ROWS_BY_TOKEN)
    ptrs = [P(8)] * 10
    assert t1(ctypes.byref(q), *ptrs, 1, P(8), P(8), 0, None) == moe.MOE_ERR_WORKSPACE
    assert t1(ctypes.byref(q), *ptrs, 2, P(8), P(8), 0, None) == moe.MOE_ERR_UNSUPPORTED
    assert t1(ctypes.byref(q), *ptrs, 1, None, P(8), 0, None) == moe.MOE_ERR_INVALID_ARG
    q.K = 2
    assert t1(ctypes.byref(q), *ptrs, 1, P(8), P(8), 0, None) == moe.MOE_ERR_INVALID_ARG
    q.K = 1; q.w_dtype = q.x_dtype = 0
    assert t1(ctypes.byref(q), *ptrs, 1, P(8), P(8), 0, None) == moe.MOE_ERR_UNSUPPORTED
    q.w_dtype = q.x_dtype = 1; q.row_layout = moe.MOE_ROWS_SORTED
    assert t1(ctypes.byref(q), *ptrs, 1, P(8), P(8), 0, None) == moe.MOE_ERR_UNSUPPORTED
    # the backward of the unpermute: H a multiple of 4, fp32 or bf16 rows, every pointer given
    ub = lib.moe_unpermute_combine_backward
    args = [P(8)] * 6
    assert ub(4, 2, 8, 16, 6, *args, 0, P(8), P(8), None) == moe.MOE_ERR_UNSUPPORTED
    assert ub(4, 2, 8, 16, 8, *args, 2, P(8), P(8), None) == moe.MOE_ERR_UNSUPPORTED
    assert ub(4, 2, 8, 16, 8, *args, 0, P(8), None, None) == moe.MOE_ERR_INVALID_ARG
    assert ub(4, 2, 8, 16, 8, None, *args[1:], 0, P(8), P(8), None) == moe.MOE_ERR_INVALID_ARG
    assert ub(4, 0, 8, 16, 8, *args, 0, P(8), P(8), None) == moe.MOE_ERR_INVALID_ARG
    assert ub(0, 2, 8, 16, 8, None, None, None, None, None, None, 0, None, None, None) == moe.MOE_OK
    # the sorted row layout: not for fp32, unknown layouts rejected, x has C rows
    p = moe._FfnParams(64, 2, 8, 256, 256, 16, 0, 0, 0, moe.MOE_ROWS_SORTED)
    assert lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(p)) == -1
    p.w_dtype = p.x_dtype = 1; p.row_layout = 7
    assert lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(p)) == -1
    p.w_dtype = 2; p.row_layout = moe.MOE_ROWS_SORTED
    ws_sorted = lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(p))
    p.row_layout = moe.MOE_ROWS_BY_TOKEN
    ws_token = lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(p))
    C = oracle.align_capacity(128, 8, 16)
    assert ws_sorted - ws_token == (C * 256 + 255) // 256 * 256 - 64 * 256 + \
        (C * 4 + 255) // 256 * 256 - (64 * 4 + 255) // 256 * 256   # x codes and scales per row


def test_schedule_validation(lib):
    P = ctypes.c_void_p
    p = moe._FfnParams(64, 2, 8, 256, 256, 16, 1, 1, 0, 0, moe.MOE_SCHEDULE_FUSED)
    two = moe._FfnParams(64, 2, 8, 256, 256, 16, 1, 1, 0, 0, moe.MOE_SCHEDULE_TWO_LAUNCH)
    # the one-stage control block: queue counters, status and two words per block
    C = oracle.align_capacity(128, 8, 16)
    extra = lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(p)) - \
        lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(two))
    assert extra == ((8 + 8 + 2 * (C // 16 + 1)) * 4 + 255) // 256 * 256
    p.schedule = 5
    assert lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(p)) == -1
    p.schedule = moe.MOE_SCHEDULE_FUSED; p.w_dtype = p.x_dtype = 0
    assert lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(p)) == -1     # not for fp32


def test_backward_validation(lib):
    P = ctypes.c_void_p
    ok = moe._FfnParams(256, 2, 8, 512, 256, 64, moe.MOE_BF16, moe.MOE_BF16, 0, 0, 0)
    assert lib.moe_ffn_backward_workspace_bytes(ctypes.byref(ok)) > 0
    for field, value in (("w_dtype", moe.MOE_FP8_E4M3), ("B", 32), ("I", 384), ("weight_layout", 1),
                         ("row_layout", 1), ("schedule", 1), ("grad_dtype", moe.MOE_FP8_E4M3)):
        p = moe._FfnParams(256, 2, 8, 512, 256, 64, moe.MOE_BF16, moe.MOE_BF16, 0, 0, 0)
        setattr(p, field, value)
        assert lib.moe_ffn_backward_workspace_bytes(ctypes.byref(p)) == -1, field
    args = [P(8)] * 17                                       # 16 arrays and the workspace
    args[8] = None                                           # expert_offsets is required here
    assert lib.moe_ffn_backward(ctypes.byref(ok), *args, 1 << 40, None) == moe.MOE_ERR_INVALID_ARG
    args[8] = P(8)
    args[10] = None                                          # gate_up may be NULL (recomputed)
    assert lib.moe_ffn_backward(ctypes.byref(ok), *args, 16, None) == moe.MOE_ERR_WORKSPACE
    # the training forward: bf16 only, by token, two launches; gate_up required
    tr = lib.moe_grouped_ffn_train
    targs = [P(8)] * 8
    assert tr(ctypes.byref(ok), *targs, P(8), 0, None) == moe.MOE_ERR_WORKSPACE
    assert tr(ctypes.byref(ok), *targs[:7], None, P(8), 0, None) == moe.MOE_ERR_INVALID_ARG
    f8 = moe._FfnParams(256, 2, 8, 512, 256, 64, moe.MOE_FP8_E4M3, moe.MOE_BF16, 0, 0, 0)
    assert tr(ctypes.byref(f8), *targs, P(8), 0, None) == moe.MOE_ERR_UNSUPPORTED
    r = moe._RouteParams(4, 8, 2, 0, 1, 1, 1, 1.0, 0)
    assert lib.moe_route_backward(ctypes.byref(r), P(8), P(8), P(8), None, None) == moe.MOE_ERR_INVALID_ARG
    r.score = 7
    assert lib.moe_route_backward(ctypes.byref(r), P(8), P(8), P(8), P(8), None) == moe.MOE_ERR_INVALID_ARG


def test_product_path_fails_loudly_without_the_library(tmp_path):
    # no fallback: with the library missing the binding raises, and it never
    # pulls in the CPU oracle
    import subprocess
    import sys
    code = ("import sys\n"
            "import routing_align_sort_amd as moe\n"
            "try:\n"
            "    moe.moe_align_sort_capacity(4, 2, 8, 16)\n"
            "    print('no error')\n"
            "except ImportError as e:\n"
            "    print('raised:', e)\n"
            "print('oracle imported' if 'oracle' in sys.modules else 'oracle not imported')\n")
    env = dict(os.environ, MOE_LIB_PATH=str(tmp_path / "missing.so"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, cwd=ROOT,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    assert "raised:" in r.stdout and "missing.so" in r.stdout, r.stdout
    assert "oracle not imported" in r.stdout


def test_product_sources_do_not_reference_the_oracle():
    pkg = os.path.join(ROOT, "routing_align_sort_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", src, re.M), f
                assert "moe_oracle" not in src, f


def test_bf16_slot_rows_are_checked_on_the_host(lib):
    # y_dtype: fp32 or bf16; bf16 only with matrix-core weights and rows by
    # slot; the training forward and the backward read fp32 slot rows
    P = ctypes.c_void_p
    p = moe._FfnParams(64, 2, 8, 256, 256, 16, moe.MOE_BF16, moe.MOE_BF16, 0, moe.MOE_ROWS_BY_TOKEN, 0, 0,
                       moe.MOE_BF16)
    assert lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(p)) > 0
    for field, value in (("y_dtype", 7), ("y_dtype", moe.MOE_FP8_E4M3), ("row_layout", moe.MOE_ROWS_SORTED)):
        q = moe._FfnParams.from_buffer_copy(p)
        setattr(q, field, value)
        assert lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(q)) == -1, (field, value)
    q = moe._FfnParams.from_buffer_copy(p)
    q.w_dtype = q.x_dtype = moe.MOE_F32
    assert lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(q)) == -1
    assert lib.moe_ffn_backward_workspace_bytes(ctypes.byref(p)) == -1
    assert lib.moe_grouped_ffn_train(ctypes.byref(p), *([P(8)] * 8), P(8), 1 << 30, None) == \
        moe.MOE_ERR_UNSUPPORTED
    # the combine of bf16 slot rows: H a multiple of 8, known dtypes only
    cs = lib.moe_combine_slots
    assert cs(4, 2, 8, 12, P(8), moe.MOE_BF16, P(8), P(8), moe.MOE_BF16, P(8), None) == moe.MOE_ERR_UNSUPPORTED
    assert cs(4, 2, 8, 16, P(8), moe.MOE_FP8_E4M3, P(8), P(8), moe.MOE_BF16, P(8), None) == \
        moe.MOE_ERR_UNSUPPORTED
    assert cs(4, 2, 8, 16, None, moe.MOE_BF16, P(8), P(8), moe.MOE_BF16, P(8), None) == moe.MOE_ERR_INVALID_ARG
    assert cs(0, 2, 8, 16, None, moe.MOE_BF16, None, None, moe.MOE_BF16, None, None) == moe.MOE_OK
    assert cs(4, 2, 8, 12, P(8), moe.MOE_F32, P(8), P(8), 5, P(8), None) == moe.MOE_ERR_UNSUPPORTED


def test_route_quantize_is_checked_on_the_host(lib):
    # routing plus the activation quantisation of an E4M3 / MXFP4 FFN: the
    # FFN's parameters must be a quantised-activation path with token rows
    # and the routing's T, the workspace the FFN's; x_quantized is 0 or 1 and
    # only for those paths
    P = ctypes.c_void_p
    rp = moe._RouteParams(64, 8, 2, 0, 1, 1, 1, 1.0, 0)
    fp = moe._FfnParams(64, 2, 8, 256, 256, 16, moe.MOE_FP8_E4M3, moe.MOE_BF16, 0, moe.MOE_ROWS_BY_TOKEN, 0, 0,
                        moe.MOE_F32, 1)
    need = lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(fp))
    assert need > 0
    rq = lib.moe_route_topk_quantize
    assert rq(ctypes.byref(rp), P(8), None, P(8), P(8), ctypes.byref(fp), P(8), P(8), need - 1, None) == \
        moe.MOE_ERR_WORKSPACE
    assert rq(ctypes.byref(rp), P(8), None, P(8), P(8), ctypes.byref(fp), None, P(8), need, None) == \
        moe.MOE_ERR_INVALID_ARG                     # x missing
    for field, value in (("T", 32), ("row_layout", moe.MOE_ROWS_SORTED)):
        q = moe._FfnParams.from_buffer_copy(fp)
        setattr(q, field, value)
        assert rq(ctypes.byref(rp), P(8), None, P(8), P(8), ctypes.byref(q), P(8), P(8), 1 << 30, None) != \
            moe.MOE_OK, (field, value)
    q = moe._FfnParams.from_buffer_copy(fp)
    q.w_dtype = q.x_dtype = moe.MOE_BF16
    q.x_quantized = 0
    assert rq(ctypes.byref(rp), P(8), None, P(8), P(8), ctypes.byref(q), P(8), P(8), 1 << 30, None) == \
        moe.MOE_ERR_INVALID_ARG                     # bf16 weights read x as it is
    q.x_quantized = 1
    assert lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(q)) == -1
    q = moe._FfnParams.from_buffer_copy(fp)
    q.x_quantized = 2
    assert lib.moe_grouped_ffn_workspace_bytes(ctypes.byref(q)) == -1
    rp0 = moe._RouteParams(0, 8, 2, 0, 1, 1, 1, 1.0, 0)
    fp0 = moe._FfnParams.from_buffer_copy(fp)
    fp0.T = 0
    assert rq(ctypes.byref(rp0), None, None, None, None, ctypes.byref(fp0), None, None, 0, None) == moe.MOE_OK
