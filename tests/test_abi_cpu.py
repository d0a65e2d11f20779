"""C-ABI checks that need no GPU: the library loads, exports every symbol the
public headers declare, agrees with the seeded generator on the parameter list,
and rejects bad arguments before launching anything."""
import ctypes as C
import os
import re

import pytest

from spatially_sharded_conv_amd import _lib as L
from spatially_sharded_conv_amd import api
from synth import param_specs, preset

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(vaep_\w+)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol():
    lib = L.load()
    declared = _header_functions()
    assert len(declared) >= 16
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == set(L.EXPORTS)


@pytest.mark.parametrize("header", ["vaep.h", "vaep_steps.h"])
@pytest.mark.parametrize("lang", ["c", "c++"])
def test_public_header_compiles_alone(header, lang, tmp_path):
    """Each public header is self-contained plain C (no torch or HIP types leak into the
    boundary): it compiles alone as strict C99 and as C++17 with warnings as errors."""
    import shutil
    import subprocess
    cc = shutil.which("gcc" if lang == "c" else "g++")
    if cc is None:
        pytest.skip("no host compiler")
    src = tmp_path / "use.c"
    src.write_text(f'#include "{header}"\nint main(void) {{ return 0; }}\n')
    std = ["-std=c99", "-pedantic"] if lang == "c" else ["-x", "c++", "-std=c++17"]
    r = subprocess.run([cc, *std, "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
                        "-I", os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_version_and_presets_match_synth():
    assert "gfx950" in api.version()
    for i in range(1, 6):
        c = api.config_preset(i)
        s = preset(i)
        assert c.family == (L.FAMILY_WAN3D if s.is_video else L.FAMILY_KL2D)
        assert c.dtype == (L.DTYPE_BF16 if s.dtype == "bf16" else L.DTYPE_F32)
        assert c.z_channels == s.z_channels
        assert tuple(c.stage_channels[:c.n_stages]) == s.stage_channels
        assert c.resnets_per_stage == s.resnets_per_stage
        assert c.norm_groups == s.norm_groups
        assert c.temporal_up_stages == s.temporal_up_stages
        assert abs(c.eps - s.eps) < 1e-12


@pytest.mark.parametrize("i", [1, 2, 5])
def test_param_list_matches_generator(i):
    lib_params = api.param_info(api.config_preset(i))
    gen = param_specs(preset(i))
    assert [(n, s) for n, s in lib_params] == [(p.name, p.shape) for p in gen]


def test_preset_out_of_range_is_invalid():
    c = L.VaepConfig()
    assert L.load().vaep_config_preset(9, C.byref(c)) == L.VAEP_ERR_INVALID_ARG
    assert "preset" in L.last_error()


def test_bad_configs_rejected():
    lib = L.load()
    c = api.config_preset(3)
    c.stage_channels[1] = 500          # not a multiple of 32 for bf16
    assert lib.vaep_param_count(C.byref(c)) == L.VAEP_ERR_UNSUPPORTED
    c = api.config_preset(3)
    c.norm_groups = 7
    assert lib.vaep_param_count(C.byref(c)) == L.VAEP_ERR_INVALID_ARG
    c = api.config_preset(5)
    c.temporal_up_stages = 4
    assert lib.vaep_param_count(C.byref(c)) == L.VAEP_ERR_INVALID_ARG
    c = api.config_preset(3)
    c.n_stages = 0
    assert lib.vaep_param_count(C.byref(c)) == L.VAEP_ERR_INVALID_ARG


def test_param_info_index_checked():
    c = api.config_preset(1)
    n = L.load().vaep_param_count(C.byref(c))
    buf = C.create_string_buffer(8)
    shape = (C.c_int64 * 5)()
    nd = C.c_int()
    assert L.load().vaep_param_info(C.byref(c), n, buf, 8, shape, C.byref(nd)) == L.VAEP_ERR_INVALID_ARG
    # truncation keeps a terminated string
    assert L.load().vaep_param_info(C.byref(c), 0, buf, 8, shape, C.byref(nd)) == 0
    assert buf.value == b"conv_in"


def test_model_create_rejects_bad_param_counts_without_gpu_work():
    c = api.config_preset(1)
    h = C.c_void_p()
    arr = (C.c_void_p * 3)()
    rc = L.load().vaep_model_create(C.byref(c), arr, 3, None, C.byref(h))
    assert rc == L.VAEP_ERR_INVALID_ARG and "expected" in L.last_error()
    assert not h.value


def test_model_switches_reject_a_null_model():
    lib = L.load()
    assert lib.vaep_model_set_norm_fold(None, 1) == L.VAEP_ERR_INVALID_ARG
    assert lib.vaep_model_set_halo_poison(None, 1) == L.VAEP_ERR_INVALID_ARG


@pytest.mark.parametrize("i", [1, 2, 3, 4])
def test_encoder_param_list_matches_generator(i):
    from synth import encoder_param_specs, preset
    cfg = preset(i)
    lc = api.make_config(cfg.family, cfg.dtype, cfg.z_channels, cfg.stage_channels, cfg.resnets_per_stage,
                         cfg.norm_groups, cfg.temporal_up_stages, cfg.eps)
    assert api.encoder_param_info(lc) == [(s.name, tuple(s.shape)) for s in encoder_param_specs(cfg)]


def test_encoder_argument_checks_without_gpu_work():
    lib = L.load()
    c = L.VaepConfig()
    assert lib.vaep_config_preset(5, C.byref(c)) == 0
    assert lib.vaep_encoder_param_count(C.byref(c)) == L.VAEP_ERR_UNSUPPORTED   # video config
    assert lib.vaep_config_preset(2, C.byref(c)) == 0
    h = C.c_void_p()
    assert lib.vaep_encoder_create(C.byref(c), None, 0, None, C.byref(h)) == L.VAEP_ERR_INVALID_ARG
    n = C.c_size_t()
    assert lib.vaep_encode_tiled_workspace_bytes(None, 1, 64, 64, 4, 4, C.byref(n)) == L.VAEP_ERR_INVALID_ARG
    assert lib.vaep_encode_tiled(None, None, 1, 64, 64, 4, 4, None, None, 0, None, None) == L.VAEP_ERR_INVALID_ARG
    assert lib.vaep_encoder_destroy(None) == 0


def test_groupnorm_merge_argument_checks():
    lib = L.load()
    assert lib.vaep_groupnorm_merge(0, 4, None, None, None, None, None, None) == L.VAEP_ERR_INVALID_ARG
    assert lib.vaep_groupnorm_merge(2, -1, None, None, None, None, None, None) == L.VAEP_ERR_INVALID_ARG
    assert lib.vaep_groupnorm_merge(2, 4, None, None, None, None, None, None) == L.VAEP_ERR_INVALID_ARG
    assert lib.vaep_model_destroy(None) == 0


def _size_query_conv(starts, h=10, cin=64, cout=64, **kw):
    lib = L.load()
    need = C.c_size_t()
    arr = (C.c_int32 * len(starts))(*starts)
    dt = kw.get("dtype", L.DTYPE_BF16)
    rc = lib.vaep_step_conv(dt, kw.get("x_dtype", dt), None, 1, 1, cin, h, 12, None, None, cout,
                            kw.get("kt", 1), 3, 3, kw.get("causal", 0), kw.get("ups", 0), None, arr,
                            len(starts) - 1, None, None, 0, C.byref(need), None)
    return rc, need.value


def test_step_size_query_needs_no_gpu():
    rc, n = _size_query_conv([0, 3, 10])
    assert rc == 0
    elems_in = 1 * (10 + 4) * 12 * 64
    assert n >= 2 * elems_in * 2


@pytest.mark.parametrize("starts,why", [([0, 3, 3, 10], "empty"), ([0, 5, 4, 10], "reversed"),
                                        ([1, 5, 10], "cover"), ([0, 5, 9], "cover")])
def test_step_rejects_bad_band_tables(starts, why):
    rc, _ = _size_query_conv(starts)
    assert rc == L.VAEP_ERR_INVALID_ARG
    assert why in L.last_error()


def test_step_rejects_unsupported_geometry():
    assert _size_query_conv([0, 10], kt=3, causal=0)[0] == L.VAEP_ERR_UNSUPPORTED
    assert _size_query_conv([0, 10], kt=3, causal=1, ups=1)[0] == L.VAEP_ERR_UNSUPPORTED
    assert _size_query_conv([0, 10], cout=6)[0] == L.VAEP_ERR_UNSUPPORTED
    assert _size_query_conv([0, 10], cout=6, dtype=L.DTYPE_F32)[0] == 0
    assert _size_query_conv([0, 10], x_dtype=L.DTYPE_F32)[0] == 0
    assert _size_query_conv([0, 10], dtype=L.DTYPE_F32, x_dtype=L.DTYPE_BF16)[0] == L.VAEP_ERR_UNSUPPORTED


def test_too_many_bands_rejected_by_steps():
    starts = list(range(0, 66))
    rc, _ = _size_query_conv(starts, h=65)
    assert rc == L.VAEP_ERR_INVALID_ARG


def test_select_axis_matches_the_oracle_policy():
    # the library's per-request axis policy against the oracle's reading of the strategy
    # page (host-only call, no device)
    from oracle import choose_axis
    for h in range(1, 13):
        for w in range(1, 13):
            for n in range(1, 14):
                assert api.select_axis(h, w, n) == choose_axis(h, w, n), (h, w, n)
    assert api.select_axis(60, 104, 4) == "width"
    assert api.select_axis(128, 128, 8) == "width"


def test_select_axis_argument_checks():
    lib = L.load()
    a = C.c_int32()
    assert lib.vaep_select_axis(8, 8, 2, None) == L.VAEP_ERR_INVALID_ARG
    assert lib.vaep_select_axis(0, 8, 2, C.byref(a)) == L.VAEP_ERR_INVALID_ARG
    assert lib.vaep_select_axis(8, 8, 0, C.byref(a)) == L.VAEP_ERR_INVALID_ARG


def test_sharded_decode_argument_checks_without_gpu_work():
    lib = L.load()
    bad = C.c_void_p(1)

    # NULL model, then NULL pointers, unknown axis and starts with auto on a NULL model
    assert lib.vaep_decode_sharded(None, bad, 1, 1, 8, 8, L.AXIS_WIDTH, None, 2, bad, bad, 0, None,
                                   None) == L.VAEP_ERR_INVALID_ARG
    assert "model" in L.last_error()


def test_tiled_entry_points_check_arguments_without_gpu_work():
    lib = L.load()
    n = C.c_size_t()
    bad = C.c_void_p(1)
    assert lib.vaep_tiled_workspace_bytes(None, 1, 1, 8, 8, 4, 3, C.byref(n)) == L.VAEP_ERR_INVALID_ARG
    assert lib.vaep_decode_tiled(None, bad, 1, 1, 8, 8, 4, 3, bad, bad, 0, None) == L.VAEP_ERR_INVALID_ARG
    assert "model" in L.last_error()
