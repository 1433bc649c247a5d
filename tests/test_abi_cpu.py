"""The C-ABI library loads, exports every entry point that include/nc.h declares, and
rejects bad arguments without touching a GPU.  CPU only (no compute calls)."""

import ctypes
import os
import re

import pytest

from dense_decoder_only_bf16_amd import nc
from dense_decoder_only_bf16_amd.inputs import TINY, D12

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nc.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nc_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(nc.LIB_PATH):
        pytest.fail("libnc.so is not built (python -m dense_decoder_only_bf16_amd.build)")
    return nc.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert set(names) == set(nc.EXPORTED), names
    for n in names:
        assert hasattr(L, n), n


def test_abi_version(L):
    assert nc.nc_abi_version() == 1


def test_timing_struct_and_bad_class(L):
    assert ctypes.sizeof(nc.nc_timing) == 32
    assert L.nc_timing_enable(99) == nc.NC_ERR_INVALID_ARG
    assert L.nc_timing_enable(-1) == nc.NC_ERR_INVALID_ARG
    assert L.nc_timing_read(None) == nc.NC_ERR_INVALID_ARG


def test_config_struct_layout():
    # 8 int32, 3 float, 1 int32 with no padding
    assert ctypes.sizeof(nc.nc_config) == 48
    assert nc.nc_config.softcap.offset == 36 and nc.nc_config.dtype.offset == 44


def _bad_cfg(**kw):
    c = nc.make_config(TINY)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("kw,code", [
    (dict(n_kv_head=0), nc.NC_ERR_INVALID_ARG),
    (dict(n_kv_head=3), nc.NC_ERR_INVALID_ARG),  # does not divide n_head = 2
    (dict(head_dim=96, d_model=192), nc.NC_ERR_UNSUPPORTED),
    (dict(d_model=100), nc.NC_ERR_INVALID_ARG),
    (dict(n_layer=0), nc.NC_ERR_INVALID_ARG),
    (dict(vocab=0), nc.NC_ERR_INVALID_ARG),
    (dict(dtype=7), nc.NC_ERR_INVALID_ARG),
    (dict(softcap=0.0), nc.NC_ERR_INVALID_ARG),
    (dict(norm_eps=-1.0), nc.NC_ERR_INVALID_ARG),
    (dict(n_head=32, d_model=2048, head_dim=64), nc.NC_ERR_UNSUPPORTED),
    (dict(d_ff=100), nc.NC_ERR_UNSUPPORTED),
])
def test_model_create_rejects_bad_config(L, kw, code):
    cfg = _bad_cfg(**kw)
    ptrs = [1] * (6 * cfg.n_layer + 2) if cfg.n_layer > 0 else [1, 1]
    with pytest.raises(nc.NcError) as e:
        nc.nc_model_create(cfg, ptrs)
    assert e.value.code == code
    assert nc.nc_last_error() != ""


def test_model_create_null_weight(L):
    cfg = nc.make_config(TINY)
    arr = (ctypes.c_void_p * (6 * cfg.n_layer + 2))(*([1] * (6 * cfg.n_layer + 1) + [None]))
    out = ctypes.c_void_p()
    code = L.nc_model_create(ctypes.byref(cfg), arr, ctypes.byref(out))
    assert code == nc.NC_ERR_INVALID_ARG and out.value is None
    code = L.nc_model_create(None, arr, ctypes.byref(out))
    assert code == nc.NC_ERR_INVALID_ARG
    code = L.nc_model_create(ctypes.byref(cfg), None, ctypes.byref(out))
    assert code == nc.NC_ERR_INVALID_ARG


def test_model_create_without_gpu_reports_device_error(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    cfg = nc.make_config(D12)
    with pytest.raises(nc.NcError) as e:
        nc.nc_model_create(cfg, [1] * (6 * cfg.n_layer + 2))
    assert e.value.code == nc.NC_ERR_DEVICE


def test_null_handles_are_rejected(L):
    out = ctypes.c_void_p()
    assert L.nc_kv_create(None, 1, 8, ctypes.byref(out)) == nc.NC_ERR_INVALID_ARG
    assert L.nc_prefill(None, None, 1, 1, None, None, None) == nc.NC_ERR_INVALID_ARG
    assert L.nc_decode_step(None, None, 1, None, None, None) == nc.NC_ERR_INVALID_ARG
    assert L.nc_decode_greedy(None, None, 1, None, None, None, None) == nc.NC_ERR_INVALID_ARG
    assert L.nc_argmax(None, 1, 1, None, None) == nc.NC_ERR_INVALID_ARG
    assert L.nc_kv_set_lens(None, None) == nc.NC_ERR_INVALID_ARG
    assert L.nc_kv_get_lens(None, None) == nc.NC_ERR_INVALID_ARG
    assert L.nc_kv_export(None, 0, None, None, None) == nc.NC_ERR_INVALID_ARG
    assert L.nc_model_set_windows(None, None) == nc.NC_ERR_INVALID_ARG
    assert L.nc_kv_copy_rows(None, None, None, None, 0, None) == nc.NC_ERR_INVALID_ARG
    assert L.nc_sample(None, 1, 1, 1.0, 0, None, None, None) == nc.NC_ERR_INVALID_ARG
    assert L.nc_model_set_extras(None, None) == nc.NC_ERR_INVALID_ARG
    L.nc_model_free(None)
    L.nc_kv_free(None)


def test_header_constants_match_binding():
    """Every #define NC_* integer in the header has the same value in the binding."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    defs = dict(re.findall(r"#define\s+(NC_[A-Z0-9_]+)\s+\(?(-?\d+)\)?", text))
    assert len(defs) >= 15
    for name, val in defs.items():
        if name == "NC_ABI_VERSION":
            assert nc.nc_abi_version() == int(val) if os.path.exists(nc.LIB_PATH) else True
            continue
        assert getattr(nc, name) == int(val), name


def test_layer_windows_helper():
    assert nc.layer_windows("SSSL", 5, 256) == [256, 256, 256, -1, 256]
    with pytest.raises(ValueError):
        nc.layer_windows("SQ", 2, 8)
    with pytest.raises(ValueError):
        nc.layer_windows("", 2, 8)


def test_extras_struct_layout():
    assert ctypes.sizeof(nc.nc_extras) == 64
    assert nc.nc_extras.smear_gate_dev.offset == 16 and nc.nc_extras.ve_dev.offset == 40
    assert nc.nc_extras.ve_channels.offset == 56
