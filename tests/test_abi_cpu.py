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


@pytest.mark.parametrize("name", ["gqa", "mla", "wide_moe", "act", "tiny", "mla_small"])
def test_cache_size_matches_oracle_bytes(lib, name):
    """rdt_cache_size is T x batch x max_seq rows of the per-token cache the
    oracle states (GQA: K and V of the kv heads; MLA: latent + rope key)."""
    from oracle import rdt_oracle
    cfg = get_config(name)
    c = rdt.make_config(cfg)
    T, max_seq = cfg["T"], 333
    elt = 4 if cfg["dtype"] == "f32" else 2
    per_tok = rdt_oracle.kv_cache_bytes_per_token(cfg, elem_bytes=elt)
    assert lib.rdt_cache_size(ctypes.byref(c), T, max_seq) == T * cfg["batch"] * max_seq * per_tok
    assert lib.rdt_cache_size(ctypes.byref(c), 0, max_seq) == 0
    assert lib.rdt_cache_size(ctypes.byref(c), T, 0) == 0
    assert lib.rdt_cache_size(None, T, max_seq) == 0


def test_mla_cache_saving_measured(lib):
    """The MLA cache the library allocates is 16x smaller than full per-head
    keys and values of the same model (the pages claim 10-20x)."""
    import json
    facts = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))
    lo, hi = facts["mla_kv_saving_range"]["value"]
    cfg = get_config("mla")
    c = rdt.make_config(cfg)
    T, max_seq = cfg["T"], 1024
    got = lib.rdt_cache_size(ctypes.byref(c), T, max_seq)
    H = cfg["n_heads"]
    full = T * cfg["batch"] * max_seq * H * ((cfg["qk_nope_head_dim"] + cfg["qk_rope_head_dim"]) + cfg["v_head_dim"]) * 2
    assert lo <= full / got <= hi


def test_decode_null_paths(lib):
    assert lib.rdt_decode_workspace_size(None, 3, 64) == 0
    assert lib.rdt_decode_step(None, None, None, None, 1, 0, None, 8, None, None, None, 0, None) == rdt.RDT_E_INVALID
    assert lib.rdt_prefill(None, None, None, None, 1, None, None, None, 8, None, 0, None) == rdt.RDT_E_INVALID
