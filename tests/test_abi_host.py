"""The C-ABI library on the host: it loads, exports every declared symbol, agrees
with the workload shapes, and its host-side validation and format helpers work.
No kernel is launched here."""
import ctypes as C
import json
import glob
import os
import re
import sys

import numpy as np
import pytest

import oracle
import synth
from prefix_cache_flow_amd import vla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    """Every function the headers under include/ declare (vla.h: the policy interface; vla_probe.h: the
    measurement probes)."""
    names = set()
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(vla_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    L = vla.lib()
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert sorted(vla.EXPORTS) == names


@pytest.mark.parametrize("i", list(range(5)) + ["joint0", "joint1"])
def test_tensor_order_and_shapes_match_workloads(i):
    cfg = synth.config(int(i[-1]), attn="joint") if isinstance(i, str) else synth.config(i)
    specs = synth.weight_specs(cfg)
    assert vla.vla_n_tensors(cfg.to_dict()) == len(specs)
    for idx, (name, shape, kind) in enumerate(specs):
        rows, cols, k = vla.vla_tensor_info(cfg.to_dict(), idx)
        want_kind = {"gain": 0, "linear": 1, "ternary": 2}[kind]
        assert k == want_kind, name
        if kind == "gain":
            assert (rows, cols) == (shape[0], 1), name
        elif kind == "ternary":
            assert (rows, cols) == (shape[0], shape[1] // 4), name
        else:
            assert (rows, cols) == shape, name


def test_ternary_pack_matches_oracle_and_roundtrips():
    rng = np.random.default_rng(0)
    q = rng.integers(-1, 2, (13, 64), dtype=np.int8)
    p = vla.vla_ternary_pack(q)
    np.testing.assert_array_equal(p, oracle.pack_ternary(q))
    np.testing.assert_array_equal(vla.vla_ternary_unpack(p, 64), q)
    bad = p.copy()
    bad[3, 2] |= 0b11000000
    with pytest.raises(vla.VlaError) as ei:
        vla.vla_ternary_unpack(bad, 64)
    assert ei.value.status == 1
    with pytest.raises(vla.VlaError):
        vla.vla_ternary_pack(np.full((2, 8), 2, dtype=np.int8))


def test_status_strings_and_config_validation():
    assert vla.vla_status_string(0) == "VLA_OK"
    assert vla.vla_status_string(6) == "VLA_ERR_DEVICE"
    cfg = synth.config(1).to_dict()
    bad = dict(cfg, Hq=7, Hkv=2)
    assert vla.vla_n_tensors(bad) == -1
    assert "multiple" in vla.vla_last_error()
    assert vla.vla_n_tensors(dict(cfg, d_p=0)) == -1
    assert vla.vla_n_tensors(dict(cfg, hd=96)) == -1
    with pytest.raises(vla.VlaError) as ei:
        vla.vla_tensor_info(cfg, 10_000)
    assert ei.value.status == 1
    # joint attention needs matching layer counts and K/V heads, and a dense prefix
    assert vla.vla_n_tensors(dict(cfg, attn="joint", L_e=4)) == -1
    assert "joint" in vla.vla_last_error()
    assert vla.vla_n_tensors(dict(cfg, attn="joint", hd_e=128)) == -1
    assert vla.vla_n_tensors(synth.config(4, attn="joint", L_e=30, Hkv_e=20, hd_e=128).to_dict()) == -1
    assert vla.vla_n_tensors(dict(cfg, attn=7)) == -1
    # shapes the row kernels or the split-K planning cannot take are refused at creation,
    # not partway through an encode or a denoise
    assert vla.vla_n_tensors(dict(cfg, d_p=8192)) == -1
    assert "d_p" in vla.vla_last_error()
    assert vla.vla_n_tensors(dict(cfg, F_e=32768)) == -1
    assert vla.vla_n_tensors(dict(cfg, F_p=32768)) == -1
    assert vla.vla_n_tensors(dict(cfg, Hq_e=128)) == -1
    assert vla.vla_n_tensors(dict(cfg, d_p=4096, F_p=16384, F_e=16384)) > 0


def test_null_and_foreign_handles_are_rejected():
    L = vla.lib()
    assert L.vla_model_destroy(None) == 3
    assert L.vla_model_destroy(C.c_void_p(0x1234)) == 3
    assert L.vla_kv_cache_release(C.c_void_p(0x5678)) == 3
    assert L.vla_kv_cache_bytes(None, 1, 1) == 0
    b, n = C.c_int32(), C.c_int32()
    assert L.vla_kv_cache_info(C.c_void_p(0x10), C.byref(b), C.byref(n)) == 3
    out = C.c_void_p()
    assert L.vla_prefix_encode(None, None, 1, 1, None, 0, None, C.byref(out), None) == 3
    assert L.vla_prefix_encode_ex(None, None, 1, 1, 1, None, None, 0, None, C.byref(out), None) == 3
    assert L.vla_prefix_encode_ex(None, None, 0, 1, 1, None, None, 0, None, None, None) == 1
    assert L.vla_probe_arm(None, 1, 4) == 3
    assert L.vla_denoise_chunk(None, None, None, 1, None, None, 0, None, None) == 3
    cfg = vla.make_config(synth.config(0).to_dict())
    assert L.vla_model_create(C.byref(cfg), None, None, C.byref(out)) == 1
    w = vla.vla_weights()
    arr = (C.c_void_p * 3)(1, 2, 3)
    w.tensors = C.cast(arr, C.POINTER(C.c_void_p))
    w.n_tensors = 3
    assert L.vla_model_create(C.byref(cfg), C.byref(w), None, C.byref(out)) == 2


def test_gemm_unit_entry_point_rejects_unknown_epilogues():
    """vla_gemm_bf16 takes VLA_GEMM_STORE, _GEGLU or _RESIDUAL; anything else is refused before any device
    call (the pointers are never dereferenced)."""
    L = vla.lib()
    x = C.c_void_p(16)
    for bad in (-1, 3, 7):
        assert L.vla_gemm_bf16(x, x, 64, 64, 64, bad, x, None) == 1
    assert "epilogue" in vla.lib().vla_last_error().decode()
    assert L.vla_gemm_bf16(None, x, 64, 64, 64, 0, x, None) == 1


def test_create_without_gpu_reports_device_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    L = vla.lib()
    cfg = synth.config(0)
    n = vla.vla_n_tensors(cfg.to_dict())
    arr = (C.c_void_p * n)(*([16] * n))
    w = vla.vla_weights()
    w.tensors = C.cast(arr, C.POINTER(C.c_void_p))
    w.n_tensors = n
    out = C.c_void_p()
    ccfg = vla.make_config(cfg.to_dict())
    assert L.vla_model_create(C.byref(ccfg), C.byref(w), None, C.byref(out)) == 6
    assert not out.value
    x = C.c_void_p(16)
    assert L.vla_quantize_rows_i8(x, 1, 1, x, x, None) == 6


def test_bench_refuses_more_than_one_gpu():
    # the benchmark measures one GPU; asking for several ends with a message and status 2, before any GPU work
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=root)
    assert r.returncode == 2
    assert "--gpus must be 1" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
