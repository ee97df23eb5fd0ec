"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, its structs match a C compiler's layout, and the host-only
entry points (validation, spectral radius) behave."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import recurrent_depth_transformer_amd as rdt
from rdt_inputs import WORKLOADS, get_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rdt.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rdt.LIB_PATH):
        rdt_build = pytest.importorskip("recurrent_depth_transformer_amd.build")
        rdt_build.build()
    return rdt.load_library()


def _declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(rdt_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported(lib):
    decl = _declared_symbols()
    assert set(decl) == set(rdt.EXPORTED_SYMBOLS)
    out = subprocess.run(["nm", "-D", "--defined-only", rdt.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (rdt_\w+)", out))
    missing = [s for s in decl if s not in exported]
    assert not missing, missing
    for s in decl:
        assert hasattr(lib, s)


def test_struct_layout_matches_c(tmp_path):
    src = tmp_path / "layout.c"
    fields = {
        "rdt_config": [f for f, _ in rdt.RdtConfig._fields_],
        "rdt_weights": rdt.WEIGHT_FIELDS,
        "rdt_aux": rdt.AUX_FIELDS,
    }
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void){"]
    for st, fs in fields.items():
        lines.append(f'printf("%zu\\n", sizeof({st}));')
        for f in fs:
            lines.append(f'printf("%zu\\n", offsetof({st}, {f}));')
    lines.append("return 0;}")
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", str(src), "-o", str(exe)], check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    i = 0
    for cls in (rdt.RdtConfig, rdt.RdtWeights, rdt.RdtAux):
        assert vals[i] == ctypes.sizeof(cls), cls
        i += 1
        for name, _ in cls._fields_:
            assert vals[i] == getattr(cls, name).offset, (cls, name)
            i += 1


def test_config_defaults(lib):
    c = rdt.RdtConfig()
    assert lib.rdt_config_default(ctypes.byref(c)) == 0
    assert c.act_threshold == pytest.approx(0.99)
    assert c.max_T == 16 and c.n_bias_rows == 1
    assert c.norm_eps == pytest.approx(1e-6) and c.rope_base == 10000.0
    assert lib.rdt_config_default(None) == rdt.RDT_E_INVALID


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_workloads_validate(lib, name):
    c = rdt.make_config(get_config(name))
    assert lib.rdt_config_validate(ctypes.byref(c)) == 0, lib.rdt_last_error()


@pytest.mark.parametrize("field,value,status", [
    ("n_kv_heads", 3, rdt.RDT_E_INVALID),       # 16 % 3 != 0
    ("top_k", 9, rdt.RDT_E_INVALID),            # more than n_experts
    ("dim", 0, rdt.RDT_E_INVALID),
    ("head_dim", 48, rdt.RDT_E_UNSUPPORTED),
    ("n_experts", 65, rdt.RDT_E_UNSUPPORTED),
    ("expert_dim", 100, rdt.RDT_E_UNSUPPORTED),
    ("dtype", 7, rdt.RDT_E_INVALID),
])
def test_validate_rejects(lib, field, value, status):
    c = rdt.make_config(get_config("gqa"))
    setattr(c, field, value)
    assert lib.rdt_config_validate(ctypes.byref(c)) == status
    assert lib.rdt_last_error().decode()


def test_spectral_radius(lib):
    A = np.array([0.5, -0.97, 0.2], np.float32)
    rho = ctypes.c_float()
    ptr = A.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    assert lib.rdt_spectral_radius(ptr, 3, ctypes.byref(rho)) == 0
    assert rho.value == pytest.approx(0.97)
    assert lib.rdt_spectral_radius(ptr, 0, ctypes.byref(rho)) == rdt.RDT_E_INVALID


def test_null_handle_paths(lib):
    assert lib.rdt_workspace_size(None, 3) == 0
    assert lib.rdt_set_graph_mode(None, 1) == rdt.RDT_E_INVALID
    lib.rdt_destroy(None)
    assert lib.rdt_version().decode().startswith("librdt")
