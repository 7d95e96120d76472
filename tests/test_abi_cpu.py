"""The C-ABI library loads, exports what include/fp4mi.h declares, and its
host-side validation returns the documented status codes without touching
a GPU (CPU only)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4mi.h")
LIB = os.environ.get("FP4MI_SANITIZED_LIB") or os.path.join(ROOT, "block_scaled_fp4_amd", "libfp4mi.so")


def declared_functions():
    src = open(HEADER).read()
    return re.findall(r"^(?:int|const char\*)\s+(\w+)\(", src, flags=re.M)


def header_constants():
    src = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"#define\s+(FP4\w*)\s+(\d+)", src)}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libfp4mi.so is not built (python __graft_entry__.py)")
    return ctypes.CDLL(LIB)


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"fp4_quantize", "fp4_dequantize", "fp4quant_encode", "fp4quant_decode",
                          "fp4_errfeedback_qdq", "mxfp4_row_to_fp8_col", "mxfp4_row_to_fp8_row",
                          "fp4_status_string",
                          "fp4_abi_version"}
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    c = header_constants()
    lib.fp4_abi_version.restype = ctypes.c_int
    assert lib.fp4_abi_version() == c["FP4MI_ABI_VERSION"]
    lib.fp4_status_string.restype = ctypes.c_char_p
    for k in ("FP4_OK", "FP4_EINVAL", "FP4_ESHAPE", "FP4_EALIGN", "FP4_EDTYPE", "FP4_EHIP",
              "FP4_EOVERLAP"):
        assert lib.fp4_status_string(c[k]) not in (None, b"unknown status")
    assert lib.fp4_status_string(999) == b"unknown status"


def test_binding_names_match_header():
    import block_scaled_fp4_amd as m
    for n in declared_functions():
        if n.startswith("fp4_status") or n == "fp4_abi_version":
            continue
        assert callable(getattr(m, n)), n


# fake, never-dereferenced device addresses: validation must reject before use
A = 0x7F0000000000
P, I, I32, I64, U64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64


def _q(lib, x=A, dtype=1, rows=4, cols=64, fmt=0, rnd=0, tmode=0, ts=A + (1 << 30),
       packed=A + (2 << 30), scales=A + (3 << 30)):
    f = lib.fp4_quantize
    f.argtypes = [P, I, I64, I64, I, I, U64, U64, I, P, P, P, P]
    return f(x, dtype, rows, cols, fmt, rnd, 0, 0, tmode, ts, packed, scales, None)


def test_quantize_validation(lib):
    c = header_constants()
    assert _q(lib, dtype=7) == c["FP4_EDTYPE"]
    assert _q(lib, fmt=5) == c["FP4_EINVAL"]
    assert _q(lib, rnd=9) == c["FP4_EINVAL"]
    assert _q(lib, tmode=3) == c["FP4_EINVAL"]
    assert _q(lib, cols=24) == c["FP4_ESHAPE"]                  # NVFP4 needs cols % 16
    assert _q(lib, fmt=1, cols=48) == c["FP4_ESHAPE"]           # MXFP4 needs cols % 32
    assert _q(lib, rows=-1) == c["FP4_ESHAPE"]
    assert _q(lib, rows=0) == c["FP4_OK"]                       # empty: no-op
    assert _q(lib, x=None) == c["FP4_EINVAL"]
    assert _q(lib, ts=None) == c["FP4_EINVAL"]
    assert _q(lib, x=A + 8) == c["FP4_EALIGN"]
    assert _q(lib, packed=A + (2 << 30) + 2) == c["FP4_EALIGN"]
    assert _q(lib, packed=A + 64) == c["FP4_EOVERLAP"]          # inside x's 512 bytes
    assert _q(lib, scales=A + (2 << 30) + 16) == c["FP4_EOVERLAP"]


def test_other_entry_points_validation(lib):
    c = header_constants()
    enc = lib.fp4quant_encode
    enc.argtypes = [P, I, I64, I64, I32, P, P, P, P]
    assert enc(A, 1, 4, 256, 48, A + (1 << 30), A + (2 << 30), A + (3 << 30), None) == c["FP4_EINVAL"]
    assert enc(A, 1, 4, 256, 2048, A + (1 << 30), A + (2 << 30), A + (3 << 30), None) == c["FP4_EINVAL"]
    assert enc(A, 1, 4, 96, 64, A + (1 << 30), A + (2 << 30), A + (3 << 30), None) == c["FP4_ESHAPE"]
    assert enc(A, 1, 4, 256, 64, A + (1 << 30), A + (1 << 30), A + (3 << 30), None) == c["FP4_EOVERLAP"]
    ex = lib.fp4quant_encode_ex
    ex.argtypes = [P, I, I64, I64, I32, I, U64, U64, P, P, P, P]
    assert ex(A, 1, 4, 256, 64, 2, 0, 0, A + (1 << 30), A + (2 << 30), A + (3 << 30), None) == c["FP4_EINVAL"]
    assert ex(A, 1, 4, 256, 48, 1, 0, 0, A + (1 << 30), A + (2 << 30), A + (3 << 30), None) == c["FP4_EINVAL"]
    assert ex(A, 1, 4, 96, 64, 1, 0, 0, A + (1 << 30), A + (2 << 30), A + (3 << 30), None) == c["FP4_ESHAPE"]
    assert ex(A, 1, 0, 256, 64, 1, 0, 0, None, None, None, None) == c["FP4_OK"]
    dec = lib.fp4quant_decode
    dec.argtypes = [P, P, P, I64, I64, I32, P, I, P]
    assert dec(A, A + 4096, A + 8192, 4, 256, 64, A + (1 << 30), 3, None) == c["FP4_EDTYPE"]
    assert dec(A, A + 4096, A + 8192, 4, 256, 64, A + 4, 1, None) == c["FP4_EALIGN"]
    ef = lib.fp4_errfeedback_qdq
    ef.argtypes = [P, I, I64, I64, P, P, I, I, U64, U64, I, P, P, P, P]
    # in place on the same dtype is allowed; a different dtype over x is not
    assert ef(A, 0, 2, 32, A + (1 << 30), A + 64, 0, 0, 0, 0, 0, A + (2 << 30), None, None,
              None) == c["FP4_EOVERLAP"]
    assert ef(A, 0, 2, 32, A + (1 << 30), A, 1, 0, 0, 0, 0, A + (2 << 30), None, None,
              None) == c["FP4_EOVERLAP"]
    assert ef(A, 0, 2, 32, A + (1 << 30), A, 0, 0, 0, 0, 0, A + (2 << 30), A + (3 << 30), None,
              None) == c["FP4_EINVAL"]                          # packed without scales
    assert ef(A, 0, 0, 32, None, A, 0, 0, 0, 0, 0, None, None, None, None) == c["FP4_OK"]
    cv = lib.mxfp4_row_to_fp8_col
    cv.argtypes = [P, P, P, I32, I64, I64, P, P, P]
    assert cv(A, A + (1 << 30), A + (2 << 30), 0, 64, 256, A + (3 << 30), A + (4 << 30), None) == c["FP4_EINVAL"]
    assert cv(A, A + (1 << 30), A + (2 << 30), 4, 64, 200, A + (3 << 30), A + (4 << 30), None) == c["FP4_ESHAPE"]
    assert cv(A, A + (1 << 30), A + (2 << 30), 4, 1 << 26, 128, A + (3 << 30), A + (4 << 30),
              None) == c["FP4_ESHAPE"]                          # tokens limited to 2^26 - 1
    assert cv(A, A + (1 << 30), A + (2 << 30), 1 << 26, 64, 128, A + (3 << 30), A + (4 << 30),
              None) == c["FP4_ESHAPE"]                          # experts limited to 2^26 - 1
    assert cv(A + 4, A + (1 << 30), A + (2 << 30), 4, 64, 256, A + (3 << 30), A + (4 << 30), None) == c["FP4_EALIGN"]
    assert cv(A, A + (1 << 30), A + (2 << 30), 4, 64, 256, A + 100, A + (4 << 30), None) == c["FP4_EOVERLAP"]
    assert cv(A, A + (1 << 30), A + (2 << 30), 4, 0, 256, A + (3 << 30), A + (4 << 30), None) == c["FP4_OK"]
    dq = lib.fp4_dequantize
    dq.argtypes = [P, P, P, I64, I64, I, P, I, P]
    assert dq(A, A + (1 << 30), A + (2 << 30), 4, 64, 0, A + 32, 1, None) == c["FP4_EOVERLAP"]
    assert dq(A, A + (1 << 30), None, 4, 64, 0, A + (3 << 30), 1, None) == c["FP4_EINVAL"]


def test_fp8_tokblk_validation(lib):
    c = header_constants()
    f = lib.mxfp4_row_to_fp8_col_tokblk
    f.argtypes = [P, P, P, I32, I64, I64, P, P, P]

    def call(packed=A, sb=A + (1 << 30), off=A + (2 << 30), E=4, T=64, H=256, out=A + (3 << 30),
             sc=A + (4 << 30)):
        return f(packed, sb, off, E, T, H, out, sc, None)

    assert call(E=0) == c["FP4_EINVAL"]
    assert call(H=200) == c["FP4_ESHAPE"]
    assert call(E=1 << 23) == c["FP4_ESHAPE"]                 # experts limited to 2^23 - 1
    assert call(T=1 << 26) == c["FP4_ESHAPE"]
    assert call(T=0) == c["FP4_OK"]
    assert call(off=None) == c["FP4_EINVAL"]
    assert call(packed=A + 4) == c["FP4_EALIGN"]
    # the scale buffer holds H (ceil(T/128) + E) floats: 256 * (1 + 4) * 4 bytes here
    assert call(out=A + (4 << 30) + 256 * 5 * 4 - 4) == c["FP4_EOVERLAP"]


def test_fp8_row_validation(lib):
    c = header_constants()
    f = lib.mxfp4_row_to_fp8_row
    f.argtypes = [P, P, I64, I64, P, P, P]

    def call(packed=A, sb=A + (1 << 30), T=4, H=256, out=A + (2 << 30), sc=A + (3 << 30)):
        return f(packed, sb, T, H, out, sc, None)

    assert call(H=200) == c["FP4_ESHAPE"]                      # H % 128
    assert call(T=-1) == c["FP4_ESHAPE"]
    assert call(T=0) == c["FP4_OK"]                            # empty: no-op
    assert call(packed=None) == c["FP4_EINVAL"]
    assert call(out=A + (2 << 30) + 4) == c["FP4_EALIGN"]      # FP8 rows need 16-byte alignment
    assert call(sb=A + (1 << 30) + 2) == c["FP4_EALIGN"]
    assert call(out=A + 16) == c["FP4_EOVERLAP"]               # output inside the codes
    assert call(sc=A + (2 << 30) + 64) == c["FP4_EOVERLAP"]    # scales inside the FP8 rows


def test_binding_raises_without_the_library(tmp_path):
    """The product path fails loudly when the HIP library is missing: a copy
    of the package without libfp4mi.so raises ImportError on import."""
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "block_scaled_fp4_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "block_scaled_fp4_amd", "__init__.py"), pkg / "__init__.py")
    p = subprocess.run([sys.executable, "-c", "import block_scaled_fp4_amd"], cwd=tmp_path,
                       capture_output=True, text=True, timeout=300)
    assert p.returncode != 0
    assert "ImportError" in p.stderr and "libfp4mi.so" in p.stderr


def test_product_code_never_reaches_the_oracle():
    """No file of the package imports or includes the oracle: there is no
    CPU fallback for any entry point."""
    pkg = os.path.join(ROOT, "block_scaled_fp4_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            path = os.path.join(dirpath, f)
            if f.endswith(".py"):
                src = open(path).read()
                assert not re.search(r"^\s*(from|import)\s+(\.*)oracle\b", src, re.M), path
                assert "importlib" not in src and "__import__" not in src, path
            elif f.endswith((".hip", ".hpp", ".h", ".cpp")):
                src = open(path).read()
                assert not re.search(r"^\s*#\s*include\s*[<\"][^>\"]*oracle", src, re.M), path


# ------------------------------------------------ randomized invalid calls
# Each case starts from a valid argument set (fake device addresses far
# apart, so nothing overlaps) and breaks exactly one documented rule; the
# call must return that rule's status without launching anything.  Run
# under ASan/UBSan by test_abi_sanitized.py.
GAP = 1 << 40


def _quantize_case(rng, c):
    fmt, dtype = int(rng.integers(2)), int(rng.integers(2))
    blk = 32 if fmt else 16
    a = dict(x=A, dtype=dtype, rows=int(rng.integers(1, 1 << 20)), cols=blk * int(rng.integers(1, 1 << 10)),
             fmt=fmt, rnd=int(rng.integers(2)), tmode=int(rng.integers(2)), ts=A + 3 * GAP,
             packed=A + GAP, scales=A + 2 * GAP)
    muts = [("dtype", int(rng.choice([-1, 2, 3, 77])), "FP4_EDTYPE"),
            ("fmt", int(rng.choice([-1, 2, 9])), "FP4_EINVAL"),
            ("rnd", int(rng.choice([-1, 2, 5])), "FP4_EINVAL"),
            ("rows", -int(rng.integers(1, 1 << 30)), "FP4_ESHAPE"),
            ("cols", a["cols"] + int(rng.choice([1, 2, 8])) if fmt == 0 else a["cols"] + 16, "FP4_ESHAPE"),
            ("rows", 1 << 40, "FP4_ESHAPE"),
            ("x", None, "FP4_EINVAL"), ("packed", None, "FP4_EINVAL"), ("scales", None, "FP4_EINVAL"),
            ("x", A + int(rng.choice([1, 2, 4, 8, 12])), "FP4_EALIGN"),
            ("packed", A + GAP + int(rng.choice([1, 2, 3])), "FP4_EALIGN"),
            ("packed", A + 16 * int(rng.integers(0, 4)), "FP4_EOVERLAP"),
            ("scales", A + GAP + 4 * int(rng.integers(0, 8)), "FP4_EOVERLAP")]
    if fmt == 0:
        muts += [("tmode", int(rng.choice([-1, 2, 4])), "FP4_EINVAL"), ("ts", None, "FP4_EINVAL"),
                 ("ts", A + 3 * GAP + 2, "FP4_EALIGN"), ("ts", A + 2 * GAP, "FP4_EOVERLAP")]
    k, v, want = muts[int(rng.integers(len(muts)))]
    a[k] = v
    return lambda lib: _q(lib, **a), c[want], (k, v)


def _encode_case(rng, c, ex):
    G = int(1 << rng.integers(4, 11))
    a = dict(x=A, dtype=int(rng.integers(2)), rows=int(rng.integers(1, 1 << 20)),
             cols=G * int(rng.integers(1, 64)), G=G, rnd=int(rng.integers(2)), p=A + GAP, s1=A + 2 * GAP,
             s2=A + 3 * GAP)
    muts = [("dtype", 5, "FP4_EDTYPE"), ("G", int(rng.choice([0, 8, 48, 100, 2048, -64])), "FP4_EINVAL"),
            ("rows", -3, "FP4_ESHAPE"), ("cols", a["cols"] + G // 2, "FP4_ESHAPE"),
            ("x", None, "FP4_EINVAL"), ("s1", None, "FP4_EINVAL"), ("s2", None, "FP4_EINVAL"),
            ("x", A + 4, "FP4_EALIGN"), ("s1", A + 2 * GAP + 1, "FP4_EALIGN"),
            ("s1", A + 3 * GAP, "FP4_EOVERLAP"), ("p", A, "FP4_EOVERLAP")]
    if ex:
        muts.append(("rnd", int(rng.choice([-1, 2, 3])), "FP4_EINVAL"))
    k, v, want = muts[int(rng.integers(len(muts)))]
    a[k] = v

    def call(lib):
        if ex:
            f = lib.fp4quant_encode_ex
            f.argtypes = [P, I, I64, I64, I32, I, U64, U64, P, P, P, P]
            return f(a["x"], a["dtype"], a["rows"], a["cols"], a["G"], a["rnd"], 1, 2, a["p"], a["s1"], a["s2"],
                     None)
        f = lib.fp4quant_encode
        f.argtypes = [P, I, I64, I64, I32, P, P, P, P]
        return f(a["x"], a["dtype"], a["rows"], a["cols"], a["G"], a["p"], a["s1"], a["s2"], None)
    return call, c[want], (k, v)


def _fp8_case(rng, c):
    T, H, E = int(rng.integers(1, 1 << 20)), 128 * int(rng.integers(1, 64)), int(rng.integers(1, 1 << 12))
    a = dict(p=A, s=A + GAP, off=A + 2 * GAP, E=E, T=T, H=H, o=A + 3 * GAP, sc=A + 4 * GAP)
    muts = [("E", int(rng.choice([0, -1])), "FP4_EINVAL"), ("E", 1 << 26, "FP4_ESHAPE"),
            ("T", -1, "FP4_ESHAPE"), ("T", 1 << 26, "FP4_ESHAPE"), ("H", H + 64, "FP4_ESHAPE"),
            ("H", 0, "FP4_ESHAPE"), ("H", 1 << 21, "FP4_ESHAPE"), ("off", None, "FP4_EINVAL"),
            ("p", None, "FP4_EINVAL"), ("sc", None, "FP4_EINVAL"), ("p", A + 8, "FP4_EALIGN"),
            ("off", A + 2 * GAP + 4, "FP4_EALIGN"), ("o", A + 3 * GAP + 2, "FP4_EALIGN"),
            ("o", A + GAP, "FP4_EOVERLAP"), ("sc", A + 3 * GAP + 128, "FP4_EOVERLAP")]
    k, v, want = muts[int(rng.integers(len(muts)))]
    a[k] = v

    def call(lib):
        f = lib.mxfp4_row_to_fp8_col
        f.argtypes = [P, P, P, I32, I64, I64, P, P, P]
        return f(a["p"], a["s"], a["off"], a["E"], a["T"], a["H"], a["o"], a["sc"], None)
    return call, c[want], (k, v)


def _fp8_tokblk_case(rng, c):
    T, H, E = int(rng.integers(1, 1 << 20)), 128 * int(rng.integers(1, 64)), int(rng.integers(1, 1 << 12))
    a = dict(p=A, s=A + GAP, off=A + 2 * GAP, E=E, T=T, H=H, o=A + 3 * GAP, sc=A + 4 * GAP)
    nsc = 4 * H * ((T + 127) // 128 + E)                       # bytes of the token-block scales
    muts = [("E", int(rng.choice([0, -1])), "FP4_EINVAL"), ("E", 1 << 23, "FP4_ESHAPE"),
            ("T", -1, "FP4_ESHAPE"), ("T", 1 << 26, "FP4_ESHAPE"), ("H", H + 64, "FP4_ESHAPE"),
            ("H", 0, "FP4_ESHAPE"), ("H", 1 << 21, "FP4_ESHAPE"), ("off", None, "FP4_EINVAL"),
            ("o", None, "FP4_EINVAL"), ("sc", None, "FP4_EINVAL"), ("s", A + GAP + 2, "FP4_EALIGN"),
            ("sc", A + 4 * GAP + 2, "FP4_EALIGN"), ("o", A + GAP, "FP4_EOVERLAP"),
            ("sc", A + 3 * GAP + T * H - 4, "FP4_EOVERLAP"),
            ("o", A + 4 * GAP + nsc - 4, "FP4_EOVERLAP")]       # FP8 bytes inside the last scales
    k, v, want = muts[int(rng.integers(len(muts)))]
    a[k] = v

    def call(lib):
        f = lib.mxfp4_row_to_fp8_col_tokblk
        f.argtypes = [P, P, P, I32, I64, I64, P, P, P]
        return f(a["p"], a["s"], a["off"], a["E"], a["T"], a["H"], a["o"], a["sc"], None)
    return call, c[want], (k, v)


def _ef_case(rng, c):
    a = dict(x=A, dtype=int(rng.integers(2)), rows=int(rng.integers(1, 1 << 20)), cols=16 * int(rng.integers(1, 512)),
             r=A + GAP, y=A + 2 * GAP, odt=int(rng.integers(2)), rnd=int(rng.integers(2)), tmode=int(rng.integers(2)),
             ts=A + 3 * GAP, p=A + 4 * GAP, s=A + 5 * GAP)
    muts = [("dtype", 3, "FP4_EDTYPE"), ("odt", -1, "FP4_EDTYPE"), ("rnd", 2, "FP4_EINVAL"),
            ("tmode", 7, "FP4_EINVAL"), ("cols", a["cols"] + 8, "FP4_ESHAPE"), ("rows", -2, "FP4_ESHAPE"),
            ("ts", None, "FP4_EINVAL"), ("y", None, "FP4_EINVAL"), ("s", None, "FP4_EINVAL"),
            ("r", A + GAP + 8, "FP4_EALIGN"), ("y", A + 2 * GAP + 4, "FP4_EALIGN"),
            ("r", A + 2 * GAP, "FP4_EOVERLAP"), ("p", A + 3 * GAP, "FP4_EOVERLAP")]
    k, v, want = muts[int(rng.integers(len(muts)))]
    a[k] = v

    def call(lib):
        f = lib.fp4_errfeedback_qdq
        f.argtypes = [P, I, I64, I64, P, P, I, I, U64, U64, I, P, P, P, P]
        return f(a["x"], a["dtype"], a["rows"], a["cols"], a["r"], a["y"], a["odt"], a["rnd"], 3, 4, a["tmode"],
                 a["ts"], a["p"], a["s"], None)
    return call, c[want], (k, v)


def test_random_invalid_arguments_are_rejected(lib):
    import numpy as np
    c = header_constants()
    rng = np.random.default_rng(2024)
    makers = [lambda: _quantize_case(rng, c), lambda: _encode_case(rng, c, False),
              lambda: _encode_case(rng, c, True), lambda: _fp8_case(rng, c), lambda: _ef_case(rng, c),
              lambda: _fp8_tokblk_case(rng, c)]
    for i in range(3000):
        call, want, what = makers[i % len(makers)]()
        got = call(lib)
        assert got == want, (i % len(makers), what, got, want)
