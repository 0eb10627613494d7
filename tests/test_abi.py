"""C-ABI checks that need no GPU: libkie.so loads, exports every function
include/kie.h declares, and validates configurations on the host."""
import ctypes
import shutil
import subprocess

import pytest

import persistent_decode_monokernel_amd as kie
from persistent_decode_monokernel_amd import _lib
from persistent_decode_monokernel_amd.engine import make_config
from kie_synth import PRESETS


def test_header_declares_the_boundary():
    names = _lib.declared_functions()
    for must in ("kie_create", "kie_prefill", "kie_decode", "kie_reset", "kie_destroy",
                 "kie_last_error", "kie_config_check", "kie_get_position"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    missing = [n for n in _lib.declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_library_exports_nothing_else_with_c_linkage():
    # the internal helpers of the runtime must not leak into the C namespace
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm is not available")
    out = subprocess.run([nm, "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {f[2] for f in (line.split() for line in out.splitlines())
                if len(f) == 3 and f[1] == "T" and not f[2].startswith("_Z")}
    assert exported == set(_lib.declared_functions()), sorted(exported ^ set(_lib.declared_functions()))


@pytest.mark.parametrize("name", sorted(PRESETS))
def test_presets_pass_host_validation(name):
    kie.config_check(PRESETS[name])


def _code(model, **kw):
    lib = _lib.load()
    c = make_config(model, **kw)
    for k, v in kw.pop("fields", {}).items():
        setattr(c, k, v)
    return lib.kie_config_check(ctypes.byref(c)), lib.kie_last_error().decode()


def _with(model, **fields):
    lib = _lib.load()
    c = make_config(model)
    for k, v in fields.items():
        setattr(c, k, v)
    rc = lib.kie_config_check(ctypes.byref(c))
    return rc, lib.kie_last_error().decode()


@pytest.mark.parametrize("fields,code", [
    ({"d_model": 100}, -1),                      # not a multiple of 8
    ({"n_heads": 6, "n_kv_heads": 4}, -1),       # heads not a multiple of kv heads
    ({"n_heads": 24, "n_kv_heads": 3}, -8),      # group of 8 not implemented
    ({"head_dim": 192}, -8),                     # wider than 16 lanes x 8
    ({"head_dim": 60}, -8),                      # not a multiple of 8
    ({"ffn_hidden": 1000 + 4}, -1),
    ({"vocab_out": 5000}, -1),                   # lm_head rows > embedding rows
    ({"max_seq": 0}, -1),
    ({"rms_eps": -1.0}, -1),
    ({"rope_base": 1.0}, -1),
    ({"flags": 0x80}, -1),
    ({"n_workgroups": -3}, -1),
    ({"timeout_ms": -1}, -1),
])
def test_invalid_configs_are_rejected(fields, code):
    rc, msg = _with(PRESETS["tiny"], **fields)
    assert rc == code, (rc, msg)
    assert msg


def test_moe_field_validation():
    m = PRESETS["moe"]
    assert _with(m, top_k=0)[0] == -1
    assert _with(m, top_k=65)[0] == -1
    assert _with(m, top_k=15, n_shared_experts=2)[0] == -8    # more than 16 active experts
    assert _with(m, expert_hidden=1404)[0] == -1


def test_lds_budget_rejects_huge_ffn():
    rc, msg = _with(PRESETS["tiny"], ffn_hidden=65536)
    assert rc == -8 and "LDS" in msg


def test_null_config_and_last_error():
    lib = _lib.load()
    assert lib.kie_config_check(None) == -1
    assert b"NULL" in lib.kie_last_error()
    assert lib.kie_config_check(ctypes.byref(make_config(PRESETS["2b"]))) == 0
    assert lib.kie_last_error() == b""


def test_null_handle_calls_are_rejected():
    lib = _lib.load()
    assert lib.kie_prefill(None, None, 1) == -1
    assert lib.kie_decode(None, 1, None, None) == -1
    assert lib.kie_reset(None) == -1
    p = ctypes.c_int32()
    assert lib.kie_get_position(None, ctypes.byref(p)) == -1
    lib.kie_destroy(None)                       # allowed


def test_sampled_decode_validates_arguments_on_the_host():
    # rejected before anything touches a device: no GPU needed
    lib = _lib.load()
    for t in (-1.0, float("nan"), float("inf")):
        rc = lib.kie_decode_sampled(None, 1, ctypes.c_uint64(1), ctypes.c_float(t), None, None)
        assert rc == -1, t  # KIE_ERR_INVALID_ARG
        assert "temperature" in lib.kie_last_error().decode()
    rc = lib.kie_decode_sampled(None, 1, ctypes.c_uint64(1), ctypes.c_float(0.7), None, None)
    assert rc == -1  # KIE_ERR_INVALID_ARG
    assert "handle" in lib.kie_last_error().decode()


def test_batched_prefill_and_gemm_validate_arguments_on_the_host():
    # rejected before anything touches a device: no GPU needed
    lib = _lib.load()
    assert lib.kie_prefill_batched(None, None, 1) == -1
    assert "NULL" in lib.kie_last_error().decode()
    for m, n, k in ((0, 64, 32), (4, 0, 32), (4, 64, 0), (4, 64, 48), (4, 64, 70000)):
        assert lib.kie_debug_gemm(None, None, None, m, n, k, 0, None) == -1, (m, n, k)
        assert "multiple of 32" in lib.kie_last_error().decode()
    # 32768 x 32768 fp16 is 2 GiB: past the product kernel's 32-bit offsets
    for m, n, k in ((4, 32768, 32768), (65536, 64, 16384 * 2)):
        assert lib.kie_debug_gemm(None, None, None, m, n, k, 0, None) == -1, (m, n, k)
        assert "2 GiB" in lib.kie_last_error().decode()


def test_stream_probe_validates_its_shape_on_the_host():
    # the depth, the load kind and the buffer-load size limit are checked
    # before any pointer is looked at
    lib = _lib.load()
    ms = ctypes.c_float()
    for depth, kind, nbytes, text in ((3, 0, 1024, "depth"), (16, 3, 1024, "kind"),
                                      (8, 2, 1 << 32, "4 GiB"), (8, 0, 1000, "multiple of 16")):
        assert lib.kie_debug_stream_ex(None, None, nbytes, 0, depth, kind, 1, ctypes.byref(ms),
                                       None) == -1, (depth, kind, nbytes)
        assert text in lib.kie_last_error().decode(), lib.kie_last_error()


def test_moe_renorm_flag_is_accepted():
    rc, msg = _with(PRESETS["moe"], flags=0x10)
    assert rc == 0, msg
