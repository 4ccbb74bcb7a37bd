"""The C-ABI library loads and exports every entry point its header declares;
argument validation that runs before any HIP call works without a GPU."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(vla_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    from vla_flow_matching_denoise_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from vla_flow_matching_denoise_amd import build
        build.build()
    return binding.lib()


def test_header_declares_the_product_calls():
    names = declared_functions()
    for n in ("vla_expert_create", "vla_denoise", "vla_set_stream", "vla_expert_destroy", "vla_last_error",
              "vla_prefill_create", "vla_prefill", "vla_prefill_destroy"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from vla_flow_matching_denoise_amd import binding
    names = declared_functions()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"
    assert set(names) == set(binding.EXPORTED)


def test_host_side_argument_errors(lib):
    from vla_flow_matching_denoise_amd import binding as B
    assert lib.vla_denoise(None, None, None, None, None, 10, None) == B.VLA_ERR_ARG
    assert "NULL" in B.vla_last_error()
    assert lib.vla_set_option(None, B.VLA_OPT_USE_GRAPH, 1) == B.VLA_ERR_ARG
    assert lib.vla_set_stream(None, None) == B.VLA_ERR_ARG
    assert lib.vla_expert_create(None, None) is None
    assert "weights" in B.vla_last_error()
    lib.vla_expert_destroy(None)                      # NULL-safe
    assert lib.vla_device_bytes(None) == 0


@pytest.mark.parametrize("field,value", [("head_dim", 96), ("hidden", 1000), ("n_kv_heads", 3),
                                         ("action_dim", 200), ("batch", 0), ("weight_dtype", 7),
                                         ("time_emb_dim", 100)])
def test_unsupported_dims_are_rejected_before_any_device_work(lib, field, value):
    from vla_flow_matching_denoise_amd import binding as B
    from vla_flow_matching_denoise_amd.expert import make_dims
    d = make_dims(2, 256, 4, 2, 64, 704, 7, 16, 32, 1)
    setattr(d, field, value)
    w = B.VlaWeights()
    assert lib.vla_expert_create(ctypes.byref(w), ctypes.byref(d)) is None
    assert B.vla_last_error() != ""


def test_mxfp4_gate_up_tier_rejects_more_than_64_rows(lib):
    """The E4M3 + MXFP4 gate_up tier has only the weight-streaming kernel:
    creation fails, before any device work, above 64 rows, and passes the dims
    check at 64."""
    from vla_flow_matching_denoise_amd import binding as B
    from vla_flow_matching_denoise_amd.expert import make_dims
    w = B.VlaWeights()
    d = make_dims(2, 256, 4, 2, 64, 704, 7, 16, 32, 5, weight_dtype="fp8_mxfp4gu")   # 80 rows
    assert lib.vla_expert_create(ctypes.byref(w), ctypes.byref(d)) is None
    assert "MXFP4" in B.vla_last_error()
    d = make_dims(2, 256, 4, 2, 64, 704, 7, 16, 32, 4, weight_dtype="fp8_mxfp4gu")   # 64 rows
    assert lib.vla_expert_create(ctypes.byref(w), ctypes.byref(d)) is None
    assert "MXFP4" not in B.vla_last_error()          # fails later, on the NULL weight pointers


def test_prefill_host_side_argument_errors(lib):
    from vla_flow_matching_denoise_amd import binding as B
    assert lib.vla_prefill(None, None, None, None) == B.VLA_ERR_ARG
    assert "NULL" in B.vla_last_error()
    assert lib.vla_prefill_set_option(None, B.VLA_OPT_USE_GRAPH, 1) == B.VLA_ERR_ARG
    assert lib.vla_prefill_set_stream(None, None) == B.VLA_ERR_ARG
    assert lib.vla_prefill_create(None, None) is None
    assert "weights" in B.vla_last_error()
    lib.vla_prefill_destroy(None)                      # NULL-safe
    assert lib.vla_prefill_device_bytes(None) == 0


@pytest.mark.parametrize("field,value", [("head_dim", 96), ("hidden", 1000), ("hidden", 8192), ("n_kv_heads", 3),
                                         ("intermediate", 100), ("prefix_len", 0), ("prefix_len", 9000),
                                         ("batch", 0), ("rms_eps", 0.0)])
def test_prefill_unsupported_dims_are_rejected_before_any_device_work(lib, field, value):
    from vla_flow_matching_denoise_amd import binding as B
    from vla_flow_matching_denoise_amd.prefill import backbone_dims
    d = backbone_dims(2, 256, 4, 2, 64, 704, 32, 1)
    setattr(d, field, value)
    w = B.VlaBackboneWeights()
    assert lib.vla_prefill_create(ctypes.byref(w), ctypes.byref(d)) is None
    assert "unsupported" in B.vla_last_error() or "must" in B.vla_last_error()


def test_prefill_e4m3_needs_multiples_of_128(lib):
    from vla_flow_matching_denoise_amd import binding as B
    from vla_flow_matching_denoise_amd.prefill import backbone_dims
    w = B.VlaBackboneWeights()
    d = backbone_dims(2, 256, 4, 2, 64, 704, 32, 1, weight_dtype="fp8_e4m3")     # I = 704: not a multiple of 128
    assert lib.vla_prefill_create(ctypes.byref(w), ctypes.byref(d)) is None
    assert "128" in B.vla_last_error()
    d = backbone_dims(2, 256, 4, 2, 64, 768, 32, 1, weight_dtype="fp8_e4m3")
    assert lib.vla_prefill_create(ctypes.byref(w), ctypes.byref(d)) is None
    assert "128" not in B.vla_last_error()          # fails later, on the NULL weight pointers
    d = backbone_dims(2, 256, 4, 2, 64, 768, 32, 1, weight_dtype=7)
    assert lib.vla_prefill_create(ctypes.byref(w), ctypes.byref(d)) is None
    assert "weight_dtype" in B.vla_last_error()


def test_header_constants_match_the_binding():
    """Every integer constant the headers define has the same value in the binding."""
    import glob
    import os
    import re
    from vla_flow_matching_denoise_amd import binding as B
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    seen = 0
    for path in glob.glob(os.path.join(root, "include", "*.h")):
        for m in re.finditer(r"#define\s+(VLA_\w+)\s+\(?(-?\d+)\)?", open(path).read()):
            name, value = m.group(1), int(m.group(2))
            assert getattr(B, name, None) == value, (path, name, value)
            seen += 1
    assert seen >= 10


def _header_struct_fields(path, name):
    """(field, kind) of `typedef struct name { ... } name;` in a header, kind
    one of int32 / float / pointer."""
    text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
    m = re.search(r"typedef struct %s \{(.*?)\} %s;" % (name, name), text, flags=re.S)
    assert m, name
    fields = []
    for decl in m.group(1).split(";"):
        decl = " ".join(decl.split())
        if not decl:
            continue
        field = re.findall(r"[A-Za-z_]\w*", decl)[-1]
        kind = "pointer" if "*" in decl else ("float" if decl.startswith("float") else "int32")
        if kind == "int32":
            assert decl.startswith("int32_t"), decl
        fields.append((field, kind))
    return fields


def _ctypes_fields(cls):
    kinds = {ctypes.c_int32: "int32", ctypes.c_float: "float"}
    return [(n, kinds.get(t, "pointer" if (t is ctypes.c_void_p or hasattr(t, "contents")) else repr(t)))
            for n, t in cls._fields_]


@pytest.mark.parametrize("header, struct, cls", [
    ("vla_expert.h", "vla_dims", "VlaDims"),
    ("vla_expert.h", "vla_weights", "VlaWeights"),
    ("vla_prefill.h", "vla_backbone_dims", "VlaBackboneDims"),
    ("vla_prefill.h", "vla_backbone_weights", "VlaBackboneWeights"),
])
def test_binding_structs_match_the_header_layouts(header, struct, cls):
    """The binding's ctypes structures list the header structs' fields in the
    same order with the same kinds, so the C library reads what Python
    wrote."""
    from vla_flow_matching_denoise_amd import binding as B
    want = _header_struct_fields(os.path.join(ROOT, "include", header), struct)
    got = _ctypes_fields(getattr(B, cls))
    assert got == want
