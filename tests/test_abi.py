"""Host-side checks of libmoefp8.so (no GPU needed): the library loads, exports
every entry point the header declares, sizes workspaces, and rejects bad
arguments with the documented status before launching anything."""
import ctypes
import os
import re

import pytest

from sparse_moe_ffn_sigmoid_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moefp8.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from sparse_moe_ffn_sigmoid_amd import build
        build.build()
    return _lib.load()


def _declared():
    text = open(HEADER).read()
    return set(re.findall(r"^MOE_API\s+[\w\s\*]+?\b(\w+)\s*\(", text, flags=re.M))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert names == set(_lib.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(-3) == b"MOE_ERR_WORKSPACE"
    assert lib.moe_status_string(7) == b"MOE_ERR_UNKNOWN"


def _cfg(**kw):
    base = dict(hidden=7168, inter=2048, n_experts=256, top_k=8, n_shared=1, inter_shared=2048, n_group=8,
                topk_group=4, group_score=0, routed_scale=1.0, scale_fmt=0, norm_eps=1e-6)
    base.update(kw)
    return _lib.MoeCfgC(**base)


def test_workspace_sizes(lib):
    c = _cfg()
    n64 = lib.moe_ffn_workspace_size(64, ctypes.byref(c))
    n4k = lib.moe_ffn_workspace_size(4096, ctypes.byref(c))
    assert n64 > 0 and n4k > 60 * n64 // 2
    # fp32 sorted-row outputs dominate: T*k*d*4 bytes
    assert n4k >= 4096 * 8 * 7168 * 4
    assert lib.moe_ffn_workspace_size(-1, ctypes.byref(c)) == 0
    bad = _cfg(n_group=7)
    assert lib.moe_ffn_workspace_size(64, ctypes.byref(bad)) == 0
    dense = _cfg(n_experts=0, top_k=0, inter=0, inter_shared=18432)
    assert lib.moe_ffn_workspace_size(4096, ctypes.byref(dense)) >= 4096 * 18432
    assert lib.moe_ffn_workspace_size(64, ctypes.byref(_cfg(scale_fmt=3))) == 0
    assert lib.moe_ffn_workspace_size(64, ctypes.byref(_cfg(norm_eps=-1.0))) == 0
    assert lib.moe_ffn_workspace_size(64, ctypes.byref(_cfg(scale_fmt=1))) == n64
    assert lib.moe_permute_workspace_size(4096, 8, 256) == 32 * 256 * 4
    assert lib.moe_permute_workspace_size(10, 8, 2000) == 0


FAKE = ctypes.c_void_p(0x10000)          # aligned non-null: never dereferenced (checks fail first)


def _err(lib):
    return lib.moe_last_error().decode()


def test_quant_argument_checks(lib):
    F = _lib.MOE_SCALE_F32
    assert lib.fp8_quant_1x128(FAKE, 1, 4, 100, 100, FAKE, 100, FAKE, F, None) == _lib.MOE_ERR_UNSUPPORTED_SHAPE
    assert "multiple of 128" in _err(lib)
    assert lib.fp8_quant_1x128(FAKE, 5, 4, 128, 128, FAKE, 128, FAKE, F, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.fp8_quant_1x128(None, 1, 4, 128, 128, FAKE, 128, FAKE, F, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.fp8_quant_1x128(FAKE, 1, 4, 128, 64, FAKE, 128, FAKE, F, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.fp8_quant_1x128(ctypes.c_void_p(0x10008), 1, 4, 128, 128, FAKE, 128, FAKE, F, None) == \
        _lib.MOE_ERR_INVALID_ARG
    assert lib.fp8_quant_1x128(FAKE, 1, 4, 128, 128, FAKE, 128, FAKE, 2, None) == _lib.MOE_ERR_INVALID_ARG  # format
    assert lib.fp8_quant_1x128(None, 1, 0, 128, 128, None, 128, None, F, None) == _lib.MOE_OK   # empty: no-op
    assert lib.fp8_quant_128x128(FAKE, 130, 128, FAKE, FAKE, F, None) == _lib.MOE_ERR_UNSUPPORTED_SHAPE
    assert lib.fp8_quant_128x128(FAKE, 128, 128, FAKE, FAKE, -1, None) == _lib.MOE_ERR_INVALID_ARG


def test_rmsnorm_quant_argument_checks(lib):
    F, U = _lib.MOE_SCALE_F32, _lib.MOE_SCALE_UE8M0
    f = lib.fp8_rmsnorm_quant_1x128
    assert f(FAKE, FAKE, 1e-6, 4, 200, 200, None, 0, FAKE, 200, FAKE, F, None) == _lib.MOE_ERR_UNSUPPORTED_SHAPE
    assert f(FAKE, FAKE, -1.0, 4, 256, 256, None, 0, FAKE, 256, FAKE, F, None) == _lib.MOE_ERR_INVALID_ARG   # eps < 0
    assert f(FAKE, FAKE, float("nan"), 4, 256, 256, None, 0, FAKE, 256, FAKE, F, None) == _lib.MOE_ERR_INVALID_ARG
    assert f(FAKE, None, 1e-6, 4, 256, 256, None, 0, FAKE, 256, FAKE, U, None) == _lib.MOE_ERR_INVALID_ARG  # gamma
    assert f(FAKE, FAKE, 1e-6, 4, 256, 256, FAKE, 128, FAKE, 256, FAKE, F, None) == _lib.MOE_ERR_INVALID_ARG  # ld_y
    assert f(FAKE, FAKE, 1e-6, 4, 256, 256, None, 0, FAKE, 256, FAKE, 7, None) == _lib.MOE_ERR_INVALID_ARG
    assert f(None, None, 1e-6, 0, 256, 256, None, 0, None, 256, None, F, None) == _lib.MOE_OK               # empty


def test_bias_update_argument_checks(lib):
    f = lib.moe_bias_update
    assert f(FAKE, 4, 8, 2000, 0.01, FAKE, None, None) == _lib.MOE_ERR_UNSUPPORTED_SHAPE
    assert f(FAKE, 4, 0, 16, 0.01, FAKE, None, None) == _lib.MOE_ERR_INVALID_ARG
    assert f(FAKE, 4, 8, 16, float("inf"), FAKE, None, None) == _lib.MOE_ERR_INVALID_ARG
    assert f(FAKE, 4, 8, 16, 0.01, None, None, None) == _lib.MOE_ERR_INVALID_ARG
    assert f(None, 4, 8, 16, 0.01, FAKE, None, None) == _lib.MOE_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,code", [
    (dict(n_group=7), _lib.MOE_ERR_UNSUPPORTED_SHAPE),          # 256 % 7 != 0
    (dict(topk_group=9), _lib.MOE_ERR_INVALID_ARG),             # > n_group
    (dict(top_k=200), _lib.MOE_ERR_INVALID_ARG),                # > topk_group * E / n_group
    (dict(topk_group=1, top_k=33), _lib.MOE_ERR_INVALID_ARG),   # > 1 * 32
    (dict(n_experts=2048, n_group=8), _lib.MOE_ERR_UNSUPPORTED_SHAPE),
    (dict(group_score=3), _lib.MOE_ERR_INVALID_ARG),
])
def test_route_config_checks(lib, kw, code):
    c = _cfg(**kw)
    assert lib.moe_route(FAKE, FAKE, None, 4, ctypes.byref(c), FAKE, 0, FAKE, FAKE, None) == code


def test_route_needs_router_weights_without_given_scores(lib):
    c = _cfg()
    assert lib.moe_route(None, None, None, 4, ctypes.byref(c), FAKE, 0, FAKE, FAKE, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_route(None, None, None, 0, ctypes.byref(c), None, 0, None, None, None) == _lib.MOE_OK
    assert lib.moe_route(FAKE, FAKE, None, 4, ctypes.byref(c), FAKE, 8, FAKE, FAKE, None) == _lib.MOE_ERR_INVALID_ARG


def test_pack_checks(lib):
    assert lib.moe_pack_weights(FAKE, 1, 24, 128, ctypes.c_void_p(0x20000), None) == _lib.MOE_ERR_UNSUPPORTED_SHAPE
    assert lib.moe_pack_weights(FAKE, 1, 16, 128, FAKE, None) == _lib.MOE_ERR_INVALID_ARG      # aliased
    assert lib.moe_pack_weights(None, 0, 16, 128, None, None) == _lib.MOE_OK                   # empty


def test_permute_checks(lib):
    assert lib.moe_permute(FAKE, 4, 2, 2000, FAKE, FAKE, FAKE, None, 0, None, FAKE, 1 << 20, None) == \
        _lib.MOE_ERR_UNSUPPORTED_SHAPE
    assert lib.moe_permute(FAKE, 4, 2, 16, FAKE, FAKE, FAKE, FAKE, 0, None, FAKE, 1 << 20, None) == \
        _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_permute(FAKE, 4, 2, 16, FAKE, FAKE, FAKE, FAKE, 24, FAKE, FAKE, 1 << 20, None) == \
        _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_permute(FAKE, 4096, 8, 256, FAKE, FAKE, FAKE, None, 0, None, FAKE, 100, None) == \
        _lib.MOE_ERR_WORKSPACE


def test_gemm_checks(lib):
    epi = _lib.MoeEpiC(None, None, None)
    args = [FAKE, FAKE, None, FAKE, FAKE, FAKE]
    assert lib.fp8_grouped_gemm_blockscaled(*args, 4, 64, 200, 128, 0, ctypes.byref(epi), FAKE, None) == \
        _lib.MOE_ERR_UNSUPPORTED_SHAPE
    assert lib.fp8_grouped_gemm_blockscaled(*args, 4, 64, 384, 128, 2, ctypes.byref(epi), FAKE, None) == \
        _lib.MOE_ERR_INVALID_ARG                                    # SwiGLU needs N % 256 and h_s
    assert lib.fp8_grouped_gemm_blockscaled(*args, 0, 64, 256, 128, 0, ctypes.byref(epi), FAKE, None) == \
        _lib.MOE_ERR_UNSUPPORTED_SHAPE
    assert lib.fp8_grouped_gemm_blockscaled(*args, 4, 64, 256, 128, 9, ctypes.byref(epi), FAKE, None) == \
        _lib.MOE_ERR_INVALID_ARG
    bad = _lib.MoeEpiC(FAKE.value, None, None, 5)
    assert lib.fp8_grouped_gemm_blockscaled(*args, 4, 64, 256, 128, 2, ctypes.byref(bad), FAKE, None) == \
        _lib.MOE_ERR_INVALID_ARG                                    # unknown scale format


def test_forward_checks(lib):
    c = _cfg()
    w = _lib.MoeWeightsC(*([0x10000] * 10))
    need = lib.moe_ffn_workspace_size(64, ctypes.byref(c))
    assert lib.moe_ffn_forward(FAKE, 64, ctypes.byref(c), ctypes.byref(w), FAKE, need - 1, FAKE, None, None, None, 0,
                               None) == _lib.MOE_ERR_WORKSPACE
    assert lib.moe_ffn_forward(FAKE, 64, ctypes.byref(c), ctypes.byref(w), ctypes.c_void_p(0x10010), need, FAKE, None,
                               None, None, 0, None) == _lib.MOE_ERR_WORKSPACE                   # not 256-aligned
    assert lib.moe_ffn_forward(FAKE, 64, ctypes.byref(c), ctypes.byref(w), FAKE, need, FAKE, None, None, None, 0x10,
                               None) == _lib.MOE_ERR_INVALID_ARG                                # unknown flag
    w0 = _lib.MoeWeightsC(*([0x10000] * 2 + [0] * 8))
    assert lib.moe_ffn_forward(FAKE, 64, ctypes.byref(c), ctypes.byref(w0), FAKE, need, FAKE, None, None, None, 0,
                               None) == _lib.MOE_ERR_INVALID_ARG                                # no expert weights
    assert lib.moe_ffn_forward(FAKE, 64, ctypes.byref(c), ctypes.byref(w), FAKE, need, FAKE, None, None, None, 1,
                               None) == _lib.MOE_ERR_INVALID_ARG                                # scores given but NULL
    dense_bad = _cfg(n_experts=0, n_shared=0)
    assert lib.moe_ffn_forward(FAKE, 64, ctypes.byref(dense_bad), ctypes.byref(w), FAKE, need, FAKE, None, None, None,
                               0, None) == _lib.MOE_ERR_INVALID_ARG
    assert lib.moe_ffn_forward(None, 0, ctypes.byref(c), ctypes.byref(w), None, 0, None, None, None, None, 0, None) == \
        _lib.MOE_OK
    wn = _lib.MoeWeightsC(*([0x10000] * 10 + [0x10008]))                                    # norm_w misaligned
    assert lib.moe_ffn_forward(FAKE, 64, ctypes.byref(c), ctypes.byref(wn), FAKE, need, FAKE, None, None, None, 0,
                               None) == _lib.MOE_ERR_INVALID_ARG


def test_invalid_data_status_and_switch(lib, monkeypatch):
    assert lib.moe_status_string(_lib.MOE_ERR_INVALID_DATA) == b"MOE_ERR_INVALID_DATA"
    for val, on in ((None, 0), ("", 0), ("0", 0), ("1", 1), ("yes", 1)):
        if val is None:
            monkeypatch.delenv("MOEFP8_VALIDATE", raising=False)
        else:
            monkeypatch.setenv("MOEFP8_VALIDATE", val)
        assert lib.moe_validation_enabled() == on, val


# Calls whose arguments pass the host checks, so that each reaches its first device step.  They run
# in a child process that sees no GPU (HIP_VISIBLE_DEVICES=-1), where that step fails with
# MOE_ERR_HIP and the message names it: the validation check with MOEFP8_VALIDATE set, the call's
# own launch without.  Nothing runs on a device (the child exits early if one is visible anyway).
_PLUMBING = r'''
import ctypes, os, sys
n = ctypes.c_int(0)
if ctypes.CDLL("libamdhip64.so").hipGetDeviceCount(ctypes.byref(n)) == 0 and n.value > 0:
    print("SKIP a device is visible"); sys.exit(0)
from sparse_moe_ffn_sigmoid_amd import _lib
lib = _lib.load()
F = ctypes.c_void_p(0x100000)
def cfg(**kw):
    base = dict(hidden=7168, inter=2048, n_experts=256, top_k=8, n_shared=1, inter_shared=2048, n_group=8,
                topk_group=4, group_score=0, routed_scale=1.0, scale_fmt=0, norm_eps=1e-6)
    base.update(kw)
    return _lib.MoeCfgC(**base)
c = cfg()
w = _lib.MoeWeightsC(*([0x100000] * 10))
epi = _lib.MoeEpiC(None, F.value, None, 0)
need = lib.moe_ffn_workspace_size(64, ctypes.byref(c))
calls = {
    "moe_permute": lambda: lib.moe_permute(F, 4, 2, 8, F, F, F, None, 0, None, F, 1 << 20, None),
    "moe_unpermute": lambda: lib.moe_unpermute(F, 0, F, None, None, 4, 2, 16, F, None),
    "fp8_grouped_gemm_blockscaled": lambda: lib.fp8_grouped_gemm_blockscaled(
        F, F, F, F, F, F, 4, 64, 256, 128, 3, ctypes.byref(epi), F, None),
    "fp8_quant_128x1_grouped": lambda: lib.fp8_quant_128x1_grouped(F, 1, 64, 128, 128, F, 2, F, F, 384, F, 0, None),
    "fp8_grouped_gemm_wgrad": lambda: lib.fp8_grouped_gemm_wgrad(F, F, F, F, F, 2, 64, 128, 128, 384, F, 0, None),
    "moe_route": lambda: lib.moe_route(None, None, F, 4, ctypes.byref(c), F, 1, F, F, None),
    "moe_ffn_forward": lambda: lib.moe_ffn_forward(F, 64, ctypes.byref(c), ctypes.byref(w), F, need, F, F, None,
                                                   None, 1, None),
}
for name, call in calls.items():
    for val in ("1", "0"):
        os.environ["MOEFP8_VALIDATE"] = val
        st = call()
        print(name, val, st, lib.moe_last_error().decode())
'''


def test_validation_runs_before_the_launches():
    import subprocess
    import sys
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1", PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", _PLUMBING], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    if r.stdout.startswith("SKIP"):
        pytest.skip("a GPU is visible to the child process")
    rows = [ln.split(" ", 3) for ln in r.stdout.strip().splitlines()]
    assert len(rows) == 14, r.stdout
    for name, val, st, msg in rows:
        assert int(st) == _lib.MOE_ERR_HIP, (name, val, st, msg)
        if val == "1":
            assert msg.startswith("MOEFP8_VALIDATE check"), (name, msg)
        else:
            assert not msg.startswith("MOEFP8_VALIDATE"), (name, msg)


def test_header_compiles_as_c99_and_links_against_the_library(tmp_path):
    """The boundary is a C ABI: the header compiles as strict C99, and a C program that calls
    the host-only entry points links against the library and runs (no GPU call is made)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi.c"
    src.write_text(
        '#include <stdio.h>\n#include "moefp8.h"\n'
        "int main(void) {\n"
        "  moe_cfg_t c = {7168, 2048, 256, 8, 1, 2048, 8, 4, MOE_GROUP_SCORE_TOP2_SUM, 1.0f, MOE_SCALE_F32, 1e-6f};\n"
        "  size_t ws = moe_ffn_workspace_size(64, &c);\n"
        "  size_t pr = moe_padded_rows(1000, 8);\n"
        '  printf("%zu %zu %s\\n", ws, pr, moe_status_string(MOE_ERR_INVALID_DATA));\n'
        "  return ws > 0 && pr == (size_t)((1000 + 127) / 128 + 8) * 128 ? 0 : 1;\n"
        "}\n")
    exe = tmp_path / "abi"
    lib_path = os.path.join(ROOT, "sparse_moe_ffn_sigmoid_amd", "libmoefp8.so")   # the plain in-tree build
    if not os.path.exists(lib_path):
        pytest.skip("the in-tree library is not built")
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", f"-I{os.path.join(ROOT, 'include')}",
                        str(src), lib_path, f"-Wl,-rpath,{os.path.dirname(lib_path)}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout, r.stderr)
    assert r.stdout.split()[2] == "MOE_ERR_INVALID_DATA"
