"""The C ABI without a GPU: the library loads, exports every symbol include/awq.h declares,
and rejects bad arguments on the host before anything reaches the device. Fake non-NULL
pointers are used only in calls that must fail validation, so no kernel is ever launched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "awq.h")

b = pytest.importorskip("post_quantization_mean_amd.binding")

FAKE = 0x10000  # never dereferenced: every call below fails validation first
FAKE_ODD = 0x10008  # 8-byte aligned only


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(b.LIB_PATH):
        pytest.skip("library not built")
    return b.load_library()


def _declared():
    src = open(HEADER, encoding="utf-8").read()
    return sorted(set(re.findall(r"AWQ_API[^;(]*?\b(awq_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = _declared()
    assert len(names) == 17
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(b.exported_symbols()) == names
    assert lib.awq_abi_version() == 2


def test_status_strings(lib):
    for code, name in enumerate(["AWQ_OK", "AWQ_ERR_NULL", "AWQ_ERR_SHAPE", "AWQ_ERR_NO_TOKENS", "AWQ_ERR_ARG",
                                 "AWQ_ERR_UNSUPPORTED", "AWQ_ERR_WORKSPACE", "AWQ_ERR_HIP"]):
        assert lib.awq_status_string(code).decode() == name
    assert lib.awq_status_string(99).decode() == "AWQ_STATUS_UNKNOWN"


def _err(lib):
    return lib.awq_last_error().decode()


def test_act_stats_validation(lib):
    ws = lib.awq_act_stats_workspace_bytes(1, 1000, 256)
    assert ws > 0 and ws % 256 == 0
    assert lib.awq_act_stats(None, 1, 1000, 256, 256, FAKE, FAKE, ws, None) == 1
    assert "x is NULL" in _err(lib)
    assert lib.awq_act_stats(FAKE, 1, 0, 256, 256, FAKE, FAKE, ws, None) == 3
    assert lib.awq_act_stats(FAKE, 1, -5, 256, 256, FAKE, FAKE, ws, None) == 2
    assert lib.awq_act_stats(FAKE, 1, 1000, 200, 200, FAKE, FAKE, ws, None) == 2
    assert lib.awq_act_stats(FAKE, 7, 1000, 256, 256, FAKE, FAKE, ws, None) == 5
    assert lib.awq_act_stats(FAKE, 1, 1000, 256, 128, FAKE, FAKE, ws, None) == 4
    assert lib.awq_act_stats(FAKE, 1, 1000, 256, 260, FAKE, FAKE, ws, None) == 5  # pitch not 16-byte
    assert lib.awq_act_stats(FAKE + 2, 1, 1000, 256, 256, FAKE, FAKE, ws, None) == 5
    assert lib.awq_act_stats(FAKE, 1, 1000, 256, 256, None, FAKE, ws, None) == 1
    assert lib.awq_act_stats(FAKE, 1, 1000, 256, 256, FAKE, FAKE, ws - 8, None) == 6
    assert lib.awq_act_stats(FAKE, 1, 1000, 256, 256, FAKE, None, ws, None) == 6
    assert lib.awq_act_stats(FAKE, 1, 1000, 256, 256, FAKE, FAKE_ODD, ws, None) == 5
    assert lib.awq_act_stats_workspace_bytes(1, 0, 256) == 0
    assert lib.awq_act_stats_workspace_bytes(3, 10, 256) == 0


def _parts(n, rows=128, ptr=FAKE):
    return (ctypes.c_void_p * n)(*([ptr] * n)), (ctypes.c_int64 * n)(*([rows] * n))


def test_quant_and_pack_validation(lib):
    p, r = _parts(2)
    assert lib.awq_quant_delta(p, r, 2, 1, 256, 64, FAKE, 3, FAKE, None) == 5  # group 64
    assert lib.awq_quant_delta(p, r, 2, 1, 200, 128, FAKE, 3, FAKE, None) == 2
    assert lib.awq_quant_delta(p, r, 0, 1, 256, 128, FAKE, 3, FAKE, None) == 4
    p9, r9 = _parts(9)
    assert lib.awq_quant_delta(p9, r9, 9, 1, 256, 128, FAKE, 3, FAKE, None) == 4
    assert lib.awq_quant_delta(p, r, 2, 1, 256, 128, FAKE, 0, FAKE, None) == 4
    assert lib.awq_quant_delta(p, r, 2, 1, 256, 128, None, 3, FAKE, None) == 1
    pz, rz = _parts(2, rows=0)
    assert lib.awq_quant_delta(pz, rz, 2, 1, 256, 128, FAKE, 3, FAKE, None) == 2
    pn = (ctypes.c_void_p * 2)(FAKE, None)
    assert lib.awq_quant_delta(pn, r, 2, 1, 256, 128, FAKE, 3, FAKE, None) == 1
    assert lib.awq_quant_delta(None, r, 2, 1, 256, 128, FAKE, 3, FAKE, None) == 1
    assert lib.awq_quantize_pack(p, r, 2, 1, 256, 128, None, FAKE, FAKE, FAKE, None) == 1
    assert lib.awq_quantize_pack(p, r, 2, 2, 256, 128, FAKE, FAKE, FAKE, FAKE, None) == 5
    assert lib.awq_quantize_pack(p, r, 2, 1, 256, 128, FAKE, FAKE + 4, FAKE, FAKE, None) == 5


def test_gemm_and_argmin_validation(lib):
    assert lib.awq_error_tiles(600, 520) == 3 * 3
    assert lib.awq_error_tiles(256, 256) == 1
    assert lib.awq_error_tiles(0, 256) == 0
    assert lib.awq_error_sse(FAKE, 256, None, 1, 600, 256, 520, 4, FAKE, None) == 1
    assert lib.awq_error_sse(FAKE, 256, FAKE, 1, 0, 256, 520, 4, FAKE, None) == 3
    assert lib.awq_error_sse(FAKE, 256, FAKE, 1, 600, 256, 0, 4, FAKE, None) == 2
    assert lib.awq_error_sse(FAKE, 256, FAKE, 1, 600, 256, 520, 0, FAKE, None) == 4
    assert lib.awq_loss_argmin(FAKE, 9, 0, 600, 520, FAKE, 256, FAKE, FAKE, FAKE, None) == 4
    assert lib.awq_loss_argmin(None, 9, 4, 600, 520, FAKE, 256, FAKE, FAKE, FAKE, None) == 1
    assert lib.awq_candidate_scales(FAKE, 256, 0, FAKE, None) == 4
    assert lib.awq_candidate_scales(FAKE, 0, 20, FAKE, None) == 2
    assert lib.awq_candidate_scales(None, 256, 20, FAKE, None) == 1


def test_search_workspace_and_validation(lib):
    need = lib.awq_search_workspace_bytes(1, 4096, 4096, 12288, 128, 20, 20)
    delta = 20 * 12288 * 4096 * 2
    sse = 20 * 16 * 48 * 8
    assert need == delta + ((sse + 255) // 256) * 256
    assert lib.awq_search_workspace_bytes(1, 4096, 4096, 12288, 128, 20, 21) == 0
    assert lib.awq_search_workspace_bytes(1, 4096, 4096, 12288, 64, 20, 5) == 0
    p, r = _parts(1, rows=520)
    small = lib.awq_search_workspace_bytes(1, 600, 256, 520, 128, 7, 3)
    args = lambda **kw: dict(dict(x=FAKE, ld=256, p=p, r=r, n=1, dt=1, tok=600, d=256, am=FAKE, g=128, ng=7,
                                  cpp=3, cs=FAKE, lo=FAKE, bs=FAKE, bi=FAKE, ws=FAKE, wsb=small), **kw)

    def call(**kw):
        a = args(**kw)
        return lib.awq_search_scales(a["x"], a["ld"], a["p"], a["r"], a["n"], a["dt"], a["tok"], a["d"], a["am"],
                                     a["g"], a["ng"], a["cpp"], a["cs"], a["lo"], a["bs"], a["bi"], a["ws"],
                                     a["wsb"], None)
    assert call(wsb=small - 1) == 6
    assert call(ws=None) == 6
    assert call(cpp=8) == 4
    assert call(cpp=0) == 4
    assert call(ng=0) == 4
    assert call(tok=0) == 3
    assert call(am=None) == 1
    assert call(bi=None) == 1
    assert call(g=32) == 5
    assert call(ws=FAKE_ODD) == 5


def test_accumulate_finalize_validation(lib):
    ws = lib.awq_act_stats_workspace_bytes(1, 1000, 256)
    assert lib.awq_act_stats_accumulate(FAKE, 1, 1000, 256, 256, None, FAKE, ws, None) == 1
    assert lib.awq_act_stats_accumulate(FAKE, 1, 0, 256, 256, FAKE, FAKE, ws, None) == 3
    assert lib.awq_act_stats_accumulate(FAKE, 1, 1000, 256, 256, FAKE, FAKE, ws - 8, None) == 6
    assert lib.awq_act_stats_accumulate(FAKE, 9, 1000, 256, 256, FAKE, FAKE, ws, None) == 5
    assert lib.awq_act_stats_finalize(None, 256, 10, FAKE, None) == 1
    assert lib.awq_act_stats_finalize(FAKE, 0, 10, FAKE, None) == 2
    assert lib.awq_act_stats_finalize(FAKE, 256, 0, FAKE, None) == 3
    assert "no activation mean" in _err(lib)
    assert lib.awq_act_stats_finalize(FAKE, 256, -1, FAKE, None) == 2


def test_fold_and_export_validation(lib):
    assert lib.awq_fold_scales(None, 64, 1, 16, 64, FAKE, FAKE, 64, None) == 1
    assert lib.awq_fold_scales(FAKE, 64, 1, 0, 64, FAKE, FAKE, 64, None) == 2
    assert lib.awq_fold_scales(FAKE, 64, 1, 16, 0, FAKE, FAKE, 64, None) == 2
    assert lib.awq_fold_scales(FAKE, 32, 1, 16, 64, FAKE, FAKE, 64, None) == 4
    assert lib.awq_fold_scales(FAKE, 64, 1, 16, 64, FAKE, FAKE, 63, None) == 4
    assert lib.awq_fold_scales(FAKE, 64, 4, 16, 64, FAKE, FAKE, 64, None) == 5
    assert lib.awq_fold_scales(FAKE + 1, 64, 1, 16, 64, FAKE, FAKE, 64, None) == 5
    assert lib.awq_fold_scales(FAKE + 2, 64, 0, 16, 64, FAKE, FAKE, 64, None) == 5  # f32 needs 4-byte alignment
    assert lib.awq_export_fp16(None, FAKE, 4, 2, FAKE, FAKE, FAKE, None) == 1
    assert lib.awq_export_fp16(FAKE, FAKE, 4, 2, FAKE, FAKE, None, None) == 1
    assert lib.awq_export_fp16(FAKE, FAKE, 0, 2, FAKE, FAKE, FAKE, None) == 2
    assert lib.awq_export_fp16(FAKE, FAKE, 4, -1, FAKE, FAKE, FAKE, None) == 2
    assert lib.awq_export_fp16(FAKE + 2, FAKE, 4, 2, FAKE, FAKE, FAKE, None) == 5
