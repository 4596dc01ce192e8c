"""Source checks of the HIP library on the CPU: no floating-point atomics
(the combine and every reduction must sum in a fixed order, so results are
the same bits on every run), and every atomic targets an integer array."""
import os
import re

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "mixture_experts_decode_router_amd", "csrc")
INT_TYPES = {"int", "int32_t", "uint32_t", "unsigned", "int64_t", "uint64_t", "long"}
FLOAT_ATOMICS = re.compile(r"unsafeAtomicAdd|atomicAdd_system|atomic_fadd|atomic_fmin|atomic_fmax|"
                           r"global_atomic_add_f|global_atomic_pk_add|ds_add_f32|ds_add_rtn_f32|"
                           r"__hip_atomic_fetch_add|__atomic_fetch_add|\.fetch_add")
ATOMIC_CALL = re.compile(r"\batomic(Add|Sub|Max|Min|Inc|Dec|Exch|CAS|And|Or|Xor)\s*\(\s*&?\s*([A-Za-z_]\w*)")


def sources():
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp", ".h", ".cpp")):
            with open(os.path.join(CSRC, name)) as f:
                yield name, f.read()


def strip_comments(src):
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.sub(r"//[^\n]*", "", src)


def test_no_float_atomics_in_kernels():
    found = [(n, m.group(0)) for n, s in sources() for m in FLOAT_ATOMICS.finditer(strip_comments(s))]
    assert not found, found


def test_every_atomic_targets_an_integer_array():
    n_calls = 0
    for name, src in sources():
        code = strip_comments(src)
        for m in ATOMIC_CALL.finditer(code):
            var = m.group(2)
            decl = re.search(r"\b(\w+)\s*\*?\s*\b" + re.escape(var) + r"\s*\[", code)
            if decl is None:
                decl = re.search(r"\b(\w+)\s*\*\s*" + re.escape(var) + r"\b", code)
            assert decl is not None, (name, m.group(0))
            assert decl.group(1) in INT_TYPES, (name, m.group(0), decl.group(0))
            n_calls += 1
    assert n_calls >= 3   # the LDS histograms of the bucketing kernels
