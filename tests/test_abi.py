"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/*.h, and rejects invalid arguments on the host before
making any HIP call (so these run on a machine without a GPU)."""

import ctypes
import glob
import os
import re

import pytest

import post_weight_quantization_stats_amd as awq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, NULL, SHAPE, UNSUPPORTED, ALIGN, WORKSPACE = 0, 1, 2, 3, 4, 5
FAKE = 0x10000          # 16-byte aligned, never dereferenced on error paths
FAKE_MIS = 0x10004      # misaligned


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(awq_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("awq_act_stats", "awq_search_scale", "awq_quantize_pack", "awq_w4a16_gemm"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = awq.lib()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(declared_functions()) <= set(awq._SIGNATURES)


def test_version_and_status_strings():
    lib = awq.lib()
    assert lib.awq_abi_version() == 1
    assert lib.awq_status_string(0) == b"AWQ_OK"
    assert lib.awq_status_string(5) == b"AWQ_ERR_WORKSPACE"
    assert lib.awq_status_string(99) == b"AWQ_ERR_UNKNOWN"


def ws_size(op, M, N, K, bits=4, group=128, n_grid=20):
    out = ctypes.c_size_t(0)
    st = awq.lib().awq_workspace_size(op, M, N, K, bits, group, n_grid, ctypes.byref(out))
    return st, out.value


def test_workspace_sizes():
    st, b = ws_size(awq.OP_SEARCH_SCALE, 65536, 12288, 4096)
    assert st == OK
    assert b >= 12288 * 4096 * 2           # one candidate's bf16 difference operand
    assert b < 12288 * 4096 * 2 + 64 * 2 ** 20   # and no fp32 reference output
    assert ws_size(awq.OP_ACT_STATS, 256, 0, 512)[0] == OK
    assert ws_size(awq.OP_W4A16_GEMM, 0, 0, 128) == (OK, 0)
    assert ws_size(awq.OP_SEARCH_SCALE, 256, 512, 500)[0] == SHAPE
    assert ws_size(awq.OP_SEARCH_SCALE, 256, 512, 512, bits=2)[0] == UNSUPPORTED
    assert ws_size(awq.OP_SEARCH_SCALE, 256, 512, 512, group=64)[0] == UNSUPPORTED
    assert ws_size(awq.OP_SEARCH_SCALE, 256, 512, 512, n_grid=0)[0] == UNSUPPORTED
    assert ws_size(awq.OP_SEARCH_SCALE, 256, 512, 512, n_grid=65)[0] == UNSUPPORTED
    assert ws_size(awq.OP_SEARCH_SCALE, 0, 512, 512)[0] == SHAPE
    assert ws_size(99, 1, 1, 128)[0] == UNSUPPORTED
    assert awq.lib().awq_workspace_size(0, 1, 1, 8, 4, 128, 20, None) == NULL


def test_act_stats_errors():
    lib = awq.lib()
    f = lib.awq_act_stats
    assert f(None, 4, 8, FAKE, FAKE, 1 << 20, None) == NULL
    assert f(FAKE, 0, 8, FAKE, FAKE, 1 << 20, None) == SHAPE
    assert f(FAKE, 4, 12, FAKE, FAKE, 1 << 20, None) == SHAPE
    assert f(FAKE_MIS, 4, 8, FAKE, FAKE, 1 << 20, None) == ALIGN
    assert f(FAKE, 4, 8, FAKE, None, 0, None) == WORKSPACE
    assert f(FAKE, 4, 8, FAKE, FAKE, 8, None) == WORKSPACE
    assert b"workspace" in lib.awq_last_error()


def test_candidate_scales_errors():
    f = awq.lib().awq_candidate_scales
    assert f(None, 8, 20, FAKE, FAKE, FAKE, 1 << 20, None) == NULL
    assert f(FAKE, 0, 20, FAKE, FAKE, FAKE, 1 << 20, None) == SHAPE
    assert f(FAKE, 8, 0, FAKE, FAKE, FAKE, 1 << 20, None) == UNSUPPORTED
    assert f(FAKE, 8, 65, FAKE, FAKE, FAKE, 1 << 20, None) == UNSUPPORTED
    assert f(FAKE, 8, 20, FAKE_MIS, FAKE, FAKE, 1 << 20, None) == ALIGN
    assert f(FAKE, 8, 20, FAKE, FAKE, FAKE, 16, None) == WORKSPACE


def test_quantize_pack_errors():
    f = awq.lib().awq_quantize_pack
    assert f(None, 4, 128, None, 4, 128, FAKE, FAKE, FAKE, None) == NULL
    assert f(FAKE, 4, 128, None, 4, 128, None, FAKE, FAKE, None) == NULL
    assert f(FAKE, 4, 128, None, 5, 128, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    assert f(FAKE, 4, 128, None, 2, 128, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    assert f(FAKE, 4, 256, None, 4, 64, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    assert f(FAKE, 4, 200, None, 4, 128, FAKE, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, 4, 0, None, 4, 128, FAKE, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, -1, 128, None, 4, 128, FAKE, FAKE, FAKE, None) == SHAPE
    assert f(FAKE_MIS, 4, 128, None, 4, 128, FAKE, FAKE, FAKE, None) == ALIGN
    assert f(FAKE, 4, 128, FAKE_MIS, 4, 128, FAKE, FAKE, FAKE, None) == ALIGN
    # N == 0 is a valid no-op and makes no HIP call
    assert f(FAKE, 0, 128, None, 4, 128, FAKE, FAKE, FAKE, None) == OK


def test_gemm_errors():
    f = awq.lib().awq_w4a16_gemm
    args = dict(x=FAKE, M=4, N=8, K=128, q=FAKE, sc=FAKE, z=FAKE, bits=4, group=128, inv=None,
                yref=None, y=FAKE, sse=None, ws=None, wsb=0)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["x"], a["M"], a["N"], a["K"], a["q"], a["sc"], a["z"], a["bits"], a["group"],
                 a["inv"], a["yref"], a["y"], a["sse"], a["ws"], a["wsb"], None)

    assert call(x=None) == NULL
    assert call(y=None) == NULL                       # neither y nor sse
    assert call(sse=FAKE) == NULL                     # sse without y_ref
    assert call(bits=8) == UNSUPPORTED
    assert call(K=100) == SHAPE
    assert call(M=-1) == SHAPE
    assert call(x=FAKE_MIS) == ALIGN
    assert call(inv=FAKE_MIS) == ALIGN
    assert call(sse=FAKE, yref=FAKE) == WORKSPACE
    assert call(sse=FAKE, yref=FAKE, ws=FAKE, wsb=8) == WORKSPACE
    r = awq.lib().awq_reference_gemm
    assert r(None, 4, 8, 128, FAKE, FAKE, None) == NULL
    assert r(FAKE, 4, 8, 100, FAKE, FAKE, None) == SHAPE
    assert r(FAKE, 4, 8, 128, FAKE_MIS, FAKE, None) == ALIGN


def test_search_errors():
    f = awq.lib().awq_search_scale

    def call(x=FAKE, M=256, K=512, w=FAKE, N=512, bits=4, group=128, n_grid=20, ws=FAKE, wsb=1 << 40,
             best=FAKE):
        return f(x, M, K, w, N, bits, group, n_grid, FAKE, FAKE, best, FAKE, FAKE, FAKE, FAKE, ws,
                 wsb, None)

    assert call(x=None) == NULL
    assert call(best=None) == NULL
    assert call(M=0) == SHAPE
    assert call(N=0) == SHAPE
    assert call(K=384 + 8) == SHAPE
    assert call(bits=1) == UNSUPPORTED
    assert call(n_grid=0) == UNSUPPORTED
    assert call(w=FAKE_MIS) == ALIGN
    assert call(ws=None) == WORKSPACE
    need = ws_size(awq.OP_SEARCH_SCALE, 256, 512, 512)[1]
    assert call(wsb=need - 1) == WORKSPACE
    assert str(need) in awq.lib().awq_last_error().decode()


def test_python_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        awq.act_stats(torch.zeros((4, 8), dtype=torch.bfloat16))


def test_decode_gemm_errors_and_plan():
    f = awq.lib().awq_w4a16_decode_gemm
    args = dict(a=FAKE, M=4, N=128, K=4096, q=FAKE, sc=FAKE, z=FAKE, bits=4, group=128, y=FAKE,
                ws=None, wsb=0)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["a"], a["M"], a["N"], a["K"], a["q"], a["sc"], a["z"], a["bits"], a["group"],
                 a["y"], a["ws"], a["wsb"], None)

    assert call(a=None) == NULL
    assert call(y=None) == NULL
    assert call(M=65) == SHAPE                       # larger M: awq_w4a16_gemm
    assert call(M=-1) == SHAPE
    assert call(K=100) == SHAPE
    assert call(bits=2) == UNSUPPORTED
    assert call(group=64) == UNSUPPORTED
    assert call(a=FAKE_MIS) == ALIGN
    assert call(y=FAKE_MIS) == ALIGN
    assert call(M=0) == OK and call(N=0) == OK       # empty: no-op
    # Up to K = 8192 one workgroup's waves cover K: no workspace.  Beyond,
    # K is split across workgroups and the partials need workspace.
    assert awq.workspace_size(awq.OP_DECODE_GEMM, 4, 128, 4096) == 0
    assert awq.workspace_size(awq.OP_DECODE_GEMM, 16, 4096, 8192) == 0
    assert awq.workspace_size(awq.OP_DECODE_GEMM, 16, 4096, 8320) > 0
    # Up to 6 tokens, one workgroup of 8 waves covers up to 128 groups (and
    # beyond, workgroups of 128 groups halve the splits).
    assert awq.workspace_size(awq.OP_DECODE_GEMM, 4, 4096, 14336) == 0
    assert awq.workspace_size(awq.OP_DECODE_GEMM, 1, 4096, 16384) == 0
    assert awq.workspace_size(awq.OP_DECODE_GEMM, 4, 4096, 16512) >= 2 * 4 * 4096 * 4
    assert awq.workspace_size(awq.OP_DECODE_GEMM, 6, 4096, 14336) == 0
    assert awq.workspace_size(awq.OP_DECODE_GEMM, 7, 4096, 8320) >= 2 * 7 * 4096 * 4
    # Above 8 tokens the plan takes the fewest workgroups that fill the chip,
    # with no K split where one workgroup's 64 groups can cover K.
    assert awq.workspace_size(awq.OP_DECODE_GEMM, 17, 4096, 4096) == 0
    assert awq.workspace_size(awq.OP_DECODE_GEMM, 64, 4096, 8192) == 0
    assert awq.workspace_size(awq.OP_DECODE_GEMM, 17, 4096, 8320) >= 2 * 17 * 4096 * 4
    # A layer too narrow to fill the chip splits K further: 4096 x 14336 at
    # 16 tokens takes 4 splits of 28 groups (64 workgroups of 64 columns each).
    assert awq.workspace_size(awq.OP_DECODE_GEMM, 16, 4096, 14336) >= 4 * 16 * 4096 * 4
    need = awq.workspace_size(awq.OP_DECODE_GEMM, 4, 128, 32768)
    assert need >= 2 * 4 * 128 * 4
    assert awq.workspace_size(awq.OP_DECODE_GEMM, 7, 128, 32768) >= 4 * 7 * 128 * 4
    assert call(K=32768) == WORKSPACE
    assert call(K=32768, ws=FAKE, wsb=need - 1) == WORKSPACE


def test_dequant_operand_errors():
    f = awq.lib().awq_dequant_operand
    assert f(None, 4, 128, None, None, 4, 128, FAKE, None) == NULL
    assert f(FAKE, 4, 128, None, None, 4, 128, None, None) == NULL
    assert f(FAKE, 4, 128, None, None, 5, 128, FAKE, None) == UNSUPPORTED
    assert f(FAKE, 4, 100, None, None, 4, 128, FAKE, None) == SHAPE
    assert f(FAKE, -1, 128, None, None, 4, 128, FAKE, None) == SHAPE
    assert f(FAKE, 4, 128, FAKE_MIS, None, 4, 128, FAKE, None) == ALIGN
    assert f(FAKE, 4, 128, None, None, 4, 128, FAKE_MIS, None) == ALIGN
    assert f(None, 0, 128, None, None, 4, 128, None, None) == OK


def test_diff_operand_errors():
    f = awq.lib().awq_diff_operand
    assert f(None, 4, 128, None, None, 4, 128, FAKE, None) == NULL
    assert f(FAKE, 4, 128, None, None, 4, 128, None, None) == NULL
    assert f(FAKE, 4, 128, None, None, 5, 128, FAKE, None) == UNSUPPORTED
    assert f(FAKE, 4, 100, None, None, 4, 128, FAKE, None) == SHAPE
    assert f(FAKE, -1, 128, None, None, 4, 128, FAKE, None) == SHAPE
    assert f(FAKE, 4, 128, FAKE_MIS, None, 4, 128, FAKE, None) == ALIGN
    assert f(FAKE, 4, 128, None, None, 4, 128, FAKE_MIS, None) == ALIGN
    assert f(None, 0, 128, None, None, 4, 128, None, None) == OK


def test_candidate_sse_errors():
    f = awq.lib().awq_candidate_sse
    assert f(FAKE, 4, 8, 128, FAKE, FAKE, None, FAKE, 1 << 20, None) == NULL
    assert f(None, 4, 8, 128, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == NULL
    assert f(FAKE, 4, 8, 100, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == SHAPE
    assert f(FAKE, -1, 8, 128, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == SHAPE
    assert f(FAKE_MIS, 4, 8, 128, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == ALIGN
    assert f(FAKE, 4, 8, 128, FAKE, FAKE, FAKE + 4, FAKE, 1 << 20, None) == ALIGN
    assert f(FAKE, 4, 8, 128, FAKE, FAKE, FAKE, None, 0, None) == WORKSPACE
    assert f(FAKE, 4, 8, 128, FAKE, FAKE, FAKE, FAKE, 8, None) == WORKSPACE


def test_search_gram_errors_and_workspace():
    f = awq.lib().awq_search_scale_gram

    def call(x=FAKE, M=256, K=512, w=FAKE, N=512, bits=4, group=128, n_grid=20, ws=FAKE, wsb=1 << 40,
             best=FAKE):
        return f(x, M, K, w, N, bits, group, n_grid, FAKE, FAKE, best, FAKE, FAKE, FAKE, FAKE, ws,
                 wsb, None)

    assert call(x=None) == NULL
    assert call(best=None) == NULL
    assert call(M=0) == SHAPE
    assert call(N=0) == SHAPE
    assert call(K=384 + 8) == SHAPE
    assert call(M=(1 << 22) + 1) == SHAPE          # padded token count above the limit
    assert call(bits=1) == UNSUPPORTED
    assert call(n_grid=65) == UNSUPPORTED
    assert call(w=FAKE_MIS) == ALIGN
    assert call(ws=None) == WORKSPACE
    need = ws_size(awq.OP_SEARCH_SCALE_GRAM, 256, 512, 512)[1]
    assert call(wsb=need - 1) == WORKSPACE
    assert str(need) in awq.lib().awq_last_error().decode()
    # the workspace holds X^T (padded), G in fp32, both split operands and D
    M, N, K = 65536, 12288, 4096
    st, b = ws_size(awq.OP_SEARCH_SCALE_GRAM, M, N, K)
    assert st == OK
    core = K * M * 2 + K * K * 4 + K * 2 * K * 2 + N * 2 * K * 2 + N * K * 4
    assert core <= b < core + 64 * 2 ** 20
    assert ws_size(awq.OP_SEARCH_SCALE_GRAM, 300, 200, 384)[1] >= 384 * 384 * 2
    assert ws_size(awq.OP_SEARCH_SCALE_GRAM, 256, 512, 500)[0] == SHAPE


def test_dense_int3_entry_errors():
    pk = awq.lib().awq_quantize_pack3
    assert pk(None, 4, 128, None, 128, FAKE, FAKE, FAKE, None) == NULL
    assert pk(FAKE, 4, 128, None, 128, None, FAKE, FAKE, None) == NULL
    assert pk(FAKE, 4, 100, None, 128, FAKE, FAKE, FAKE, None) == SHAPE
    assert pk(FAKE, 4, 128, None, 64, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    assert pk(FAKE, 4, 128, None, 128, FAKE + 2, FAKE, FAKE, None) == ALIGN
    assert pk(FAKE_MIS, 4, 128, None, 128, FAKE, FAKE, FAKE, None) == ALIGN
    assert pk(None, 0, 128, None, 128, None, None, None, None) == OK
    dg = awq.lib().awq_w3a16_decode_gemm

    def call(a=FAKE, M=4, N=128, K=4096, q=FAKE, group=128, y=FAKE, ws=None, wsb=0):
        return dg(a, M, N, K, q, FAKE, FAKE, group, y, ws, wsb, None)

    assert call(a=None) == NULL
    assert call(M=65) == SHAPE
    assert call(K=100) == SHAPE
    assert call(group=64) == UNSUPPORTED
    assert call(q=FAKE + 2) == ALIGN
    assert call(K=32768) == WORKSPACE
    assert call(M=0) == OK and call(N=0) == OK


def test_decode_tiles_entry_errors():
    lib = awq.lib()
    out = ctypes.c_size_t(0)
    assert lib.awq_decode_tiles_size(40, 384, 0, 128, None) == NULL
    assert lib.awq_decode_tiles_size(40, 384, 2, 128, ctypes.byref(out)) == UNSUPPORTED
    assert lib.awq_decode_tiles_size(40, 100, 0, 128, ctypes.byref(out)) == SHAPE
    assert lib.awq_decode_tiles_size(40, 384, 0, 128, ctypes.byref(out)) == OK
    assert out.value == 48 * 384 // 2
    assert lib.awq_decode_tiles_size(40, 384, 1, 128, ctypes.byref(out)) == OK
    assert out.value == 48 * 3 * 384 // 8
    assert lib.awq_decode_tiles(None, 40, 384, 0, 128, FAKE, None) == NULL
    assert lib.awq_decode_tiles(FAKE, 40, 384, 0, 128, FAKE + 4, None) == ALIGN
    assert lib.awq_decode_tiles(FAKE, 0, 384, 0, 128, None, None) == OK
    f = lib.awq_decode_gemm_tiled
    assert f(FAKE, 4, 128, 4096, FAKE, FAKE, FAKE, 5, 128, FAKE, None, 0, None) == UNSUPPORTED
    assert f(FAKE, 65, 128, 4096, FAKE, FAKE, FAKE, 0, 128, FAKE, None, 0, None) == SHAPE
    assert f(None, 4, 128, 4096, FAKE, FAKE, FAKE, 0, 128, FAKE, None, 0, None) == NULL
    assert f(FAKE, 4, 128, 4096, FAKE + 4, FAKE, FAKE, 0, 128, FAKE, None, 0, None) == ALIGN
    # tiles beyond 4 GiB cannot be addressed
    assert f(FAKE, 4, 1 << 22, 1 << 13, FAKE, FAKE, FAKE, 0, 128, FAKE, FAKE, 1 << 40, None) == SHAPE


def test_block_op_errors():
    lib = awq.lib()
    assert lib.awq_rmsnorm(None, 4, 128, FAKE, ctypes.c_double(1e-5), FAKE, None, None) == NULL
    assert lib.awq_rmsnorm(FAKE, 4, 100, FAKE, ctypes.c_double(1e-5), FAKE, None, None) == SHAPE
    assert lib.awq_rmsnorm(FAKE, 4, 128, FAKE, ctypes.c_double(-1.0), FAKE, None, None) == UNSUPPORTED
    assert lib.awq_rmsnorm(FAKE_MIS, 4, 128, FAKE, ctypes.c_double(1e-5), FAKE, None, None) == ALIGN
    assert lib.awq_rmsnorm(None, 0, 128, None, ctypes.c_double(1e-5), None, None, None) == OK
    assert lib.awq_silu_mul(None, 4, 128, FAKE, None) == NULL
    assert lib.awq_silu_mul(FAKE, 4, 126, FAKE, None) == SHAPE
    assert lib.awq_silu_mul(FAKE, 4, 128, FAKE + 4, None) == ALIGN
    assert lib.awq_divide_rows(FAKE, 4, 3, None, FAKE, None) == NULL
    assert lib.awq_divide_rows(FAKE, 4, 3, FAKE + 2, FAKE, None) == ALIGN
    assert lib.awq_divide_rows(None, 0, 3, None, None, None) == OK
    assert lib.awq_residual_add(FAKE, None, 4, 128, FAKE, None) == NULL
    assert lib.awq_residual_add(FAKE, FAKE, 4, 12, FAKE, None) == SHAPE
    assert lib.awq_residual_add(FAKE, FAKE_MIS, 4, 128, FAKE, None) == ALIGN


def test_compact_format_entry_errors():
    lib = awq.lib()
    pk = lib.awq_quantize_pack16

    def pack(w=FAKE, N=4, K=256, s=None, bits=4, group=128, layout=0, q=FAKE, st=FAKE, z=FAKE):
        return pk(w, N, K, s, bits, group, layout, q, st, z, None)

    assert pack(w=None) == NULL and pack(st=None) == NULL and pack(z=None) == NULL
    assert pack(layout=2) == UNSUPPORTED
    assert pack(layout=1, bits=4) == UNSUPPORTED
    assert pack(bits=5) == UNSUPPORTED and pack(group=64) == UNSUPPORTED
    assert pack(K=100) == SHAPE and pack(N=-1) == SHAPE
    assert pack(st=FAKE + 1) == ALIGN
    assert pack(q=FAKE + 4) == ALIGN                  # nibble codes: 16-byte
    assert pack(w=FAKE_MIS) == ALIGN
    assert pack(N=0, w=None, q=None, st=None, z=None) == OK
    ex = lib.awq_expand_meta16
    assert ex(None, FAKE, 4, 256, 128, FAKE, FAKE, None) == NULL
    assert ex(FAKE, FAKE, 4, 100, 128, FAKE, FAKE, None) == SHAPE
    assert ex(FAKE + 1, FAKE, 4, 256, 128, FAKE, FAKE, None) == ALIGN
    assert ex(FAKE, FAKE, 4, 256, 128, FAKE + 2, FAKE, None) == ALIGN
    assert ex(None, None, 0, 256, 128, None, None, None) == OK
    f = lib.awq_decode_gemm_tiled16

    def dec(a=FAKE, M=4, N=128, K=4096, t=FAKE, st=FAKE, z=FAKE, layout=0, group=128, y=FAKE,
            ws=None, wsb=0):
        return f(a, M, N, K, t, st, z, layout, group, y, ws, wsb, None)

    assert dec(layout=5) == UNSUPPORTED
    assert dec(st=None) == NULL and dec(a=None) == NULL and dec(z=None) == NULL
    assert dec(M=65) == SHAPE and dec(K=100) == SHAPE
    assert dec(st=FAKE + 1) == ALIGN and dec(t=FAKE + 4) == ALIGN
    assert dec(K=32768) == WORKSPACE
    assert dec(N=1 << 22, K=1 << 13, ws=FAKE, wsb=1 << 40) == SHAPE
    assert dec(M=0) == OK and dec(N=0) == OK


def test_metadata_tiles_entry_errors():
    lib = awq.lib()
    out = ctypes.c_size_t(0)
    size = lib.awq_decode_meta_size
    assert size(40, 384, 128, None) == NULL
    assert size(40, 100, 128, ctypes.byref(out)) == SHAPE
    assert size(40, 384, 64, ctypes.byref(out)) == UNSUPPORTED
    assert size(-1, 384, 128, ctypes.byref(out)) == SHAPE
    assert size(40, 384, 128, ctypes.byref(out)) == OK and out.value == 3 * 16 * 3 * 4
    assert size(0, 384, 128, ctypes.byref(out)) == OK and out.value == 0
    mk = lib.awq_decode_meta
    assert mk(None, FAKE, 40, 384, 128, FAKE, None) == NULL
    assert mk(FAKE, FAKE, 40, 384, 128, None, None) == NULL
    assert mk(FAKE + 1, FAKE, 40, 384, 128, FAKE, None) == ALIGN
    assert mk(FAKE, FAKE, 40, 384, 128, FAKE + 2, None) == ALIGN
    assert mk(FAKE, FAKE, 40, 100, 128, FAKE, None) == SHAPE
    assert mk(None, None, 0, 384, 128, None, None) == OK
    f = lib.awq_decode_gemm_tiled_meta

    def dec(a=FAKE, M=4, N=128, K=4096, t=FAKE, m=FAKE, layout=0, group=128, y=FAKE, ws=None,
            wsb=0):
        return f(a, M, N, K, t, m, layout, group, y, ws, wsb, None)

    assert dec(layout=5) == UNSUPPORTED and dec(group=64) == UNSUPPORTED
    assert dec(m=None) == NULL and dec(a=None) == NULL and dec(t=None) == NULL and dec(y=None) == NULL
    assert dec(M=65) == SHAPE and dec(K=100) == SHAPE and dec(N=-1) == SHAPE
    assert dec(m=FAKE + 2) == ALIGN and dec(t=FAKE + 4) == ALIGN and dec(a=FAKE_MIS) == ALIGN
    assert dec(layout=1, t=FAKE + 2) == ALIGN                        # dense INT3 tiles: 4-byte
    assert dec(K=32768) == WORKSPACE
    assert dec(N=1 << 22, K=1 << 13, ws=FAKE, wsb=1 << 40) == SHAPE
    assert dec(M=0) == OK and dec(N=0) == OK


def test_ceiling_entry_errors():
    lib = awq.lib()
    flops = ctypes.c_int64(0)
    m = lib.awq_ceiling_mfma
    assert m(0, 10, 0, FAKE, ctypes.byref(flops), None) == SHAPE
    assert m(65537, 10, 0, FAKE, ctypes.byref(flops), None) == SHAPE
    assert m(4, 0, 0, FAKE, ctypes.byref(flops), None) == SHAPE
    assert m(4, (1 << 20) + 1, 0, FAKE, ctypes.byref(flops), None) == SHAPE
    assert m(4, 10, 0, None, ctypes.byref(flops), None) == NULL
    assert m(4, 10, 0, FAKE, None, None) == NULL
    assert m(4, 10, 0, FAKE + 2, ctypes.byref(flops), None) == ALIGN
    f = lib.awq_ceiling_stream

    def s(mode, src, dst, nbytes, blocks=1024):
        return f(mode, src, dst, nbytes, blocks, None)

    assert s(3, FAKE, FAKE, 4096) == UNSUPPORTED
    assert s(0, FAKE, FAKE, 0) == SHAPE and s(0, FAKE, FAKE, 4100) == SHAPE
    assert s(0, FAKE, FAKE, 4096, 0) == SHAPE and s(0, FAKE, FAKE, 4096, (1 << 24) + 1) == SHAPE
    assert s(0, None, FAKE, 4096) == NULL and s(1, None, FAKE, 4096) == NULL
    assert s(2, None, None, 4096) == NULL
    assert s(0, FAKE + 4, FAKE, 4096) == ALIGN and s(0, FAKE, FAKE + 4, 4096) == ALIGN
    assert s(1, FAKE, FAKE + 2, 4096) == ALIGN                  # the read sink: 4-byte
    assert s(2, None, FAKE + 8, 4096) == ALIGN


def test_last_error_is_per_thread():
    """Each thread sees the message of its own last failing call."""
    import threading
    lib = awq.lib()
    seen = {}

    def worker(name, call):
        for _ in range(200):
            st = call()
            msg = lib.awq_last_error()
            if name in seen and seen[name] != (st, msg):
                seen[name] = None
                return
            seen[name] = (st, msg)

    calls = {
        "shape": lambda: lib.awq_act_stats(FAKE, 4, 100, FAKE, FAKE, 1 << 20, None),
        "unsupported": lambda: lib.awq_quantize_pack(FAKE, 4, 128, None, 5, 128, FAKE, FAKE, FAKE, None),
    }
    threads = [threading.Thread(target=worker, args=(k, c)) for k, c in calls.items()]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert seen["shape"] is not None and seen["shape"][0] == SHAPE
    assert seen["unsupported"] is not None and seen["unsupported"][0] == UNSUPPORTED
    assert seen["shape"][1] != seen["unsupported"][1]


def test_staged_gemm_entry_errors():
    """awq_w4a16_gemm_staged: layout, bits, shapes, alignment and workspace
    are rejected on the host."""
    f = awq.lib().awq_w4a16_gemm_staged
    st, need = ws_size(awq.OP_W4A16_GEMM_STAGED, 300, 64, 256)
    assert st == OK and need >= 64 * 256 * 2
    args = lambda **k: dict(dict(x=FAKE, M=300, N=64, K=256, q=FAKE, sc=FAKE, ze=FAKE, bits=4,
                                 group=128, layout=0, inv=None, yref=None, y=FAKE, sse=None,
                                 ws=FAKE, wsb=need), **k)
    call = lambda a: f(a["x"], a["M"], a["N"], a["K"], a["q"], a["sc"], a["ze"], a["bits"],
                       a["group"], a["layout"], a["inv"], a["yref"], a["y"], a["sse"], a["ws"],
                       a["wsb"], None)
    assert call(args(layout=2)) == UNSUPPORTED
    assert call(args(layout=1, bits=4)) == UNSUPPORTED       # dense words hold 3-bit codes
    assert call(args(bits=5)) == UNSUPPORTED
    assert call(args(K=200)) == SHAPE
    assert call(args(x=None)) == NULL
    assert call(args(y=None)) == NULL                        # neither y nor sse
    assert call(args(y=None, sse=FAKE)) == NULL              # sse without y_ref
    assert call(args(x=FAKE_MIS)) == ALIGN
    assert call(args(q=FAKE + 2)) == ALIGN
    assert call(args(ws=None)) == WORKSPACE
    assert call(args(wsb=need - 1)) == WORKSPACE


def _cpu(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


@pytest.mark.parametrize("case", [
    "decode_out", "decode_scales_dtype", "decode_zeros_shape", "decode_qweight_cols",
    "decode3_words", "tiled_size", "tiled_scales", "tiled16_steps", "tiled16_zeros4",
    "meta_steps", "tiled_meta_size", "tiled_meta_tiles",
    "w4a16_inv_s", "w4a16_y_ref", "w4a16_scales", "w3a16_bits", "w3a16_words", "dequant_s", "divide_rows_s", "residual_y",
    "rmsnorm_gamma", "tiles_qweight", "noncontiguous"])
def test_python_wrappers_check_shapes_before_the_device(case):
    """Every wrapper checks dtype, exact shape and contiguity of each tensor
    argument before any pointer reaches the library (the kernels size their
    accesses from M, N and K, not from the allocations); on this GPU-less
    machine each mistake must be reported as itself, not as "not a GPU
    tensor"."""
    import torch
    bf, f32, u8, i32, f16 = torch.bfloat16, torch.float32, torch.uint8, torch.int32, torch.float16
    M, N, K = 4, 32, 256
    a = _cpu((M, K), bf)
    qw, sc, ze = _cpu((N, K // 8), i32), _cpu((N, 2), f32), _cpu((N, 2), u8)
    tiles = _cpu((awq.decode_tiles_size(N, K) // 4,), i32)
    calls = {
        "decode_out": (lambda: awq.decode_gemm(a, qw, sc, ze, out=_cpu((M, N - 1), f32)), "out must"),
        "decode_scales_dtype": (lambda: awq.decode_gemm(a, qw, sc.half(), ze), "scales must"),
        "decode_zeros_shape": (lambda: awq.decode_gemm(a, qw, sc, _cpu((N, 3), u8)), "zeros must"),
        "decode_qweight_cols": (lambda: awq.decode_gemm(a, _cpu((N, K // 8 - 1), i32), sc, ze),
                                "qweight must"),
        "decode3_words": (lambda: awq.decode_gemm3(a, qw, sc, ze), "qweight3 must"),
        "tiled_size": (lambda: awq.decode_gemm_tiled(a, tiles[:-4], sc, ze), "tiles must hold"),
        "tiled_scales": (lambda: awq.decode_gemm_tiled(a, tiles, _cpu((N, 3), f32), ze), "scales must"),
        "tiled16_steps": (lambda: awq.decode_gemm_tiled16(a, tiles, sc, _cpu((N, 1), u8)),
                          "steps16 must"),
        "tiled16_zeros4": (lambda: awq.decode_gemm_tiled16(a, tiles, _cpu((N, 2), f16),
                                                           _cpu((N, 2), u8)), "zeros4 must"),
        "meta_steps": (lambda: awq.decode_meta(_cpu((N, 2), f32), _cpu((N, 1), u8)),
                       "steps16 must"),
        "tiled_meta_size": (lambda: awq.decode_gemm_tiled_meta(
            a, tiles, _cpu((awq.decode_meta_size(N, K) // 4 - 1,), i32), N), "meta must"),
        "tiled_meta_tiles": (lambda: awq.decode_gemm_tiled_meta(
            a, tiles[:-4], _cpu((awq.decode_meta_size(N, K) // 4,), i32), N), "tiles must hold"),
        "w4a16_inv_s": (lambda: awq.w4a16_gemm(a, qw, sc, ze, inv_s=_cpu((K - 1,), f32)),
                        "inv_s must"),
        "w4a16_y_ref": (lambda: awq.w4a16_gemm(a, qw, sc, ze, y_ref=_cpu((M, N + 1), f32)),
                        "y_ref must"),
        "w4a16_scales": (lambda: awq.w4a16_gemm(a, qw, _cpu((N, 2), f16), ze), "scales must"),
        "w3a16_bits": (lambda: awq.w4a16_gemm(a, _cpu((N, 3 * K // 32), i32), sc, ze, 4,
                                              layout=awq.LAYOUT_INT3_DENSE), "holds 3-bit codes"),
        "w3a16_words": (lambda: awq.w4a16_gemm(a, qw, sc, ze, 3, layout=awq.LAYOUT_INT3_DENSE),
                        "qweight must"),
        "dequant_s": (lambda: awq.dequant_operand(_cpu((N, K), bf), _cpu((K + 1,), f32), None),
                      "s must"),
        "divide_rows_s": (lambda: awq.divide_rows(_cpu((N, 2), f32), _cpu((N - 1,), f32)), "s must"),
        "residual_y": (lambda: awq.residual_add(a, _cpu((M, K - 8), f32)), "y must"),
        "rmsnorm_gamma": (lambda: awq.rmsnorm(a, _cpu((K - 8,), f32)), "gamma must"),
        "tiles_qweight": (lambda: awq.decode_tiles(_cpu((N, K // 8 + 1), i32), K), "qweight must"),
        "noncontiguous": (lambda: awq.decode_gemm(a, qw, _cpu((2, N), f32).t(), ze), "contiguous"),
    }
    fn, msg = calls[case]
    with pytest.raises((ValueError, TypeError), match=msg):
        fn()
    # with every shape right, the same call fails only on the device check
    good = {"decode_out": lambda: awq.decode_gemm(a, qw, sc, ze, out=_cpu((M, N), f32)),
            "tiled_meta_size": lambda: awq.decode_gemm_tiled_meta(
                a, tiles, _cpu((awq.decode_meta_size(N, K) // 4,), i32), N),
            "tiled_size": lambda: awq.decode_gemm_tiled(a, tiles, sc, ze),
            "w3a16_bits": lambda: awq.w4a16_gemm(a, _cpu((N, 3 * K // 32), i32), sc, ze, 3,
                                                 layout=awq.LAYOUT_INT3_DENSE)}
    if case in good:
        with pytest.raises(ValueError, match="GPU tensor"):
            good[case]()


def test_noalloc_scratch_covers_every_workload_layer():
    """The entry point that allocates nothing keeps the decode contraction's
    K-split partials in a 16 MiB static scratch; the header states that this
    covers every workload layer at 1 to 64 tokens.  The partials' size is
    the decode workspace size, a host-side function of the plan."""
    import synth
    worst, where = 0, None
    for workload, layers in synth.WORKLOADS.items():
        for spec in layers:
            for M in range(1, 65):
                need = awq.workspace_size(awq.OP_DECODE_GEMM, M, spec.N, spec.K)
                assert need <= 16 << 20, (workload, spec.name, M, need)
                if need > worst:
                    worst, where = need, (workload, spec.name, M)
    # the largest is the Llama-2-70B down projection at 64 tokens: 4 K splits
    assert where == ("llama2_70b_mlp", "down", 64) and worst == 4 * 64 * 8192 * 4
