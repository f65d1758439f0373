"""C ABI: the library loads, exports every declared symbol, and validates
arguments on the host (no GPU work is enqueued by any call here)."""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_moe_transformer_glm_amd as glm
from sparse_moe_transformer_glm_amd._lib import Dims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "glm_moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(glm_moe_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("glm_moe_route", "glm_moe_forward", "glm_moe_workspace_bytes",
              "glm_moe_workspace_size", "glm_moe_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", glm.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (glm_moe_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    L = glm.lib()
    for n in declared_functions():
        assert getattr(L, n) is not None


def test_exports_are_c_linkage_only():
    out = subprocess.run(["nm", "-D", "--defined-only", glm.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    text_syms = re.findall(r"\bT (\S+)", out)
    assert [s for s in text_syms if s.startswith("glm_moe_")]
    assert not [s for s in text_syms if "glm" in s and not s.startswith("glm_moe_")], \
        "internal symbols are exported"


def test_no_undefined_internal_symbols():
    out = subprocess.run(["nm", "-D", "--undefined-only", glm.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    bad = [l for l in out.splitlines() if "glm" in l]
    assert not bad, bad


def test_peaks_library_exports_its_header():
    """The ceiling microbenchmarks live in a library of their own with their own header."""
    from sparse_moe_transformer_glm_amd import build as B
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "glm_peaks.h")).read(),
                  flags=re.S)
    declared = sorted(set(re.findall(r"\b(glm_peak_\w+)\s*\(", text)))
    assert declared == ["glm_peak_clock_probe", "glm_peak_gemm_step", "glm_peak_hbm_read",
                        "glm_peak_mfma"]
    out = subprocess.run(["nm", "-D", "--defined-only", B.PEAKS_LIB], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (glm_\w+)", out))
    assert exported == set(declared), exported


def _ws(T, D, E, F, Fs, k, dt=glm.BF16):
    n = ctypes.c_size_t(0)
    st = glm.lib().glm_moe_workspace_size(ctypes.byref(Dims(T, D, E, F, Fs, dt, dt)), k,
                                          ctypes.byref(n))
    return st, n.value


def test_workspace_bytes_matches_workspace_size():
    """glm_moe_workspace_bytes returns the size glm_moe_workspace_size writes,
    0 with an empty error for T = 0, and 0 with the cause for rejected dims."""
    L = glm.lib()
    for T, D, E, F, Fs, k, dt in ((64, 6144, 256, 2048, 2048, 8, glm.BF16),
                                  (8192, 6144, 256, 2048, 2048, 8, glm.BF16),
                                  (37, 100, 5, 30, 7, 2, glm.F32), (1, 64, 4, 64, 64, 1, glm.BF16)):
        d = Dims(T, D, E, F, Fs, dt, dt)
        n = ctypes.c_size_t(0)
        assert L.glm_moe_workspace_size(ctypes.byref(d), k, ctypes.byref(n)) == glm.OK
        assert L.glm_moe_workspace_bytes(ctypes.byref(d), k) == n.value > 0
    assert L.glm_moe_workspace_bytes(ctypes.byref(Dims(0, 128, 8, 64, 64, glm.BF16, glm.BF16)),
                                     2) == 0
    assert L.glm_moe_last_error() == b""
    for d, k in ((Dims(64, 128, 8, 64, 64, glm.BF16, glm.BF16), 9),     # top_k > E
                 (Dims(64, 128, 300, 64, 64, glm.BF16, glm.BF16), 8),   # E > 256
                 (Dims(64, 100, 8, 64, 64, glm.BF16, glm.BF16), 2)):    # D not /64 on bf16
        assert L.glm_moe_workspace_bytes(ctypes.byref(d), k) == 0
        assert L.glm_moe_last_error() != b""
    assert L.glm_moe_workspace_bytes(None, 2) == 0
    assert glm.workspace_bytes(64, 128, 8, 64, 64, 2) == glm.workspace_size(64, 128, 8, 64, 64, 2)
    with pytest.raises(glm.GlmMoeError):
        glm.workspace_bytes(64, 128, 8, 64, 64, 9)


def test_workspace_sizes():
    st, n0 = _ws(0, 6144, 256, 2048, 2048, 8)
    assert st == glm.OK and n0 == 0
    st, n1 = _ws(64, 6144, 256, 2048, 2048, 8)
    assert st == glm.OK
    # at least the fp32 slot outputs and the bf16 hidden activations
    assert n1 >= 64 * 8 * 6144 * 4 + 64 * 8 * 2048 * 2
    st, n2 = _ws(8192, 6144, 256, 2048, 2048, 8)
    assert st == glm.OK and n2 > n1
    st, n3 = _ws(64, 128, 8, 64, 64, 2, glm.F32)
    assert st == glm.OK and n3 > 0
    assert n2 % 256 == 0


@pytest.mark.parametrize("dims,k,code", [
    ((64, 6144, 257, 2048, 2048), 8, glm.EUNSUPPORTED),   # E > 256
    ((64, 6144, 256, 2048, 2048), 0, glm.EINVAL),         # top_k < 1
    ((64, 6144, 256, 2048, 2048), 33, glm.EINVAL),        # top_k > 32
    ((64, 128, 4, 64, 64), 5, glm.EINVAL),                # top_k > E
    ((64, 100, 8, 64, 64), 2, glm.EUNSUPPORTED),          # bf16 D not /64
    ((64, 128, 8, 96, 64), 2, glm.EUNSUPPORTED),          # bf16 F not /64
    ((64, 128, 8, 64, 32), 2, glm.EUNSUPPORTED),          # bf16 F_shared not /64
    ((-1, 128, 8, 64, 64), 2, glm.EINVAL),                # negative T
    ((64, 0, 8, 64, 64), 2, glm.EINVAL),                  # D = 0
])
def test_invalid_dims(dims, k, code):
    st, _ = _ws(*dims, k)
    assert st == code
    assert glm.lib().glm_moe_last_error()


def test_dtype_mix_unsupported():
    n = ctypes.c_size_t(0)
    st = glm.lib().glm_moe_workspace_size(ctypes.byref(Dims(64, 128, 8, 64, 64, glm.BF16, glm.F32)),
                                          2, ctypes.byref(n))
    assert st == glm.EUNSUPPORTED


def test_fp32_path_accepts_any_sizes():
    st, n = _ws(5, 100, 3, 30, 7, 2, glm.F32)
    assert st == glm.OK and n > 0


def _forward(d, k, ptrs, ws=0, ws_bytes=0):
    L = glm.lib()
    return L.glm_moe_forward(ctypes.byref(d), *ptrs[:9], k, 2.5, ptrs[9], None, None, ws,
                             ws_bytes, None)


FAKE = 1 << 40  # never dereferenced: validation fails before any enqueue


def test_forward_null_and_alignment_checks():
    d = Dims(64, 128, 8, 64, 64, glm.BF16, glm.BF16)
    good = [FAKE] * 10
    for i in range(10):
        p = list(good)
        p[i] = 0
        assert _forward(d, 2, p) == glm.EINVAL
    for i in range(10):
        p = list(good)
        p[i] = FAKE + 8
        assert _forward(d, 2, p) == glm.EINVAL


def test_forward_workspace_checks():
    d = Dims(64, 128, 8, 64, 64, glm.BF16, glm.BF16)
    _, need = _ws(64, 128, 8, 64, 64, 2)
    good = [FAKE] * 10
    assert _forward(d, 2, good, FAKE, need - 1) == glm.EWORKSPACE
    assert _forward(d, 2, good, 0, need) == glm.EINVAL
    assert _forward(d, 2, good, FAKE + 16, need) == glm.EINVAL  # not 256-byte aligned


def test_zero_tokens_is_a_no_op():
    d = Dims(0, 128, 8, 64, 64, glm.BF16, glm.BF16)
    assert _forward(d, 2, [0] * 10) == glm.OK
    L = glm.lib()
    assert L.glm_moe_route(ctypes.byref(d), None, None, None, 2, 2.5, None, None, None, 0,
                           None) == glm.OK


def test_route_validation():
    L = glm.lib()
    d = Dims(64, 128, 8, 64, 64, glm.BF16, glm.BF16)
    assert L.glm_moe_route(ctypes.byref(d), FAKE, FAKE, FAKE, 9, 2.5, FAKE, FAKE, FAKE, 1 << 30,
                           None) == glm.EINVAL
    assert L.glm_moe_route(None, FAKE, FAKE, FAKE, 2, 2.5, FAKE, FAKE, FAKE, 1 << 30,
                           None) == glm.EINVAL


def test_status_strings_and_version():
    L = glm.lib()
    for code in (glm.OK, glm.EINVAL, glm.EUNSUPPORTED, glm.EWORKSPACE, glm.EHIP):
        assert L.glm_moe_status_string(code)
    assert L.glm_moe_status_string(12345) == b"unknown status"
    assert L.glm_moe_version() >= 100


def test_trace_argument_checks():
    L = glm.lib()
    assert L.glm_moe_trace_create(None, 4) == glm.EINVAL
    h = ctypes.c_void_p()
    assert L.glm_moe_trace_create(ctypes.byref(h), 0) == glm.EINVAL
    assert L.glm_moe_trace_reset(None) == glm.EINVAL
    assert L.glm_moe_trace_destroy(None) == glm.OK


# ----------------------------------------------------------- options, dense

from sparse_moe_transformer_glm_amd._lib import Options  # noqa: E402


def _ws_ex(dims, k, opts, dt=glm.BF16):
    n = ctypes.c_size_t(0)
    st = glm.lib().glm_moe_workspace_size_ex(ctypes.byref(Dims(*dims, dt, dt)),
                                             None if opts is None else ctypes.byref(opts), k,
                                             ctypes.byref(n))
    return st, n.value


GLM = (64, 6144, 256, 2048, 2048)


def test_workspace_ex_defaults_match_plain():
    assert _ws_ex(GLM, 8, None) == _ws(*GLM, 8)
    assert _ws_ex(GLM, 8, Options()) == _ws(*GLM, 8)
    assert _ws_ex(GLM, 8, Options(8, 4, 2, None, 1e-5, 1)) == _ws(*GLM, 8)


def test_workspace_ex_norm_holds_the_normalised_input():
    _, plain = _ws(*GLM, 8)
    st, n = _ws_ex(GLM, 8, Options(1, 1, 0, FAKE, 1e-5, 0))
    assert st == glm.OK and n == plain + 64 * 6144 * 2
    st, n = _ws_ex((64, 128, 8, 64, 64), 2, Options(1, 1, 0, FAKE, 1e-5, 0), glm.F32)
    _, p32 = _ws(64, 128, 8, 64, 64, 2, glm.F32)
    assert st == glm.OK and n == p32 + 64 * 128 * 4


@pytest.mark.parametrize("opts,k,code", [
    (Options(65, 1, 2, None, 0.0, 0), 8, glm.EUNSUPPORTED),   # > 64 groups
    (Options(3, 1, 2, None, 0.0, 0), 8, glm.EINVAL),          # E % n_group
    (Options(-2, 1, 2, None, 0.0, 0), 8, glm.EINVAL),         # negative n_group
    (Options(8, 0, 2, None, 0.0, 0), 8, glm.EINVAL),          # topk_group < 1
    (Options(8, 9, 2, None, 0.0, 0), 8, glm.EINVAL),          # topk_group > n_group
    (Options(8, 4, 33, None, 0.0, 0), 8, glm.EINVAL),         # group_topk > group size
    (Options(8, 4, -1, None, 0.0, 0), 8, glm.EINVAL),         # group_topk < 0
    (Options(64, 1, 2, None, 0.0, 0), 8, glm.EINVAL),         # kept experts (4) < top_k
    (Options(1, 1, 0, FAKE, -1.0, 0), 8, glm.EINVAL),         # eps < 0
    (Options(1, 1, 0, FAKE, float("nan"), 0), 8, glm.EINVAL), # eps NaN
    (Options(1, 1, 0, FAKE, float("inf"), 0), 8, glm.EINVAL), # eps inf
    (Options(1, 1, 0, FAKE + 4, 1e-5, 0), 8, glm.EINVAL),     # misaligned norm weight
])
def test_invalid_options(opts, k, code):
    st, _ = _ws_ex(GLM, k, opts)
    assert st == code
    assert glm.lib().glm_moe_last_error()


def test_valid_group_options():
    for o in (Options(8, 4, 2, None, 0.0, 0), Options(64, 2, 1, None, 0.0, 0),
              Options(1, 0, 0, None, 0.0, 0), Options(0, 0, 0, None, 0.0, 0),
              Options(8, 1, 0, None, 0.0, 0), Options(256, 1, 1, None, 0.0, 0)):
        st, _ = _ws_ex((64, 128, 64 if o.n_group <= 64 else 256, 64, 64), 1, o)
        assert st == (glm.OK if o.n_group <= 64 else glm.EUNSUPPORTED), (o.n_group, st)


def _forward_ex(d, opts, k, ptrs, ws=0, ws_bytes=0):
    return glm.lib().glm_moe_forward_ex(ctypes.byref(d), opts and ctypes.byref(opts), *ptrs[:9],
                                        k, 1.0, ptrs[9], None, None, ws, ws_bytes, None, None)


def test_forward_ex_checks_like_forward():
    d = Dims(64, 128, 8, 64, 64, glm.BF16, glm.BF16)
    o = Options(4, 2, 2, None, 0.0, 1)
    good = [FAKE] * 10
    for i in range(10):
        p = list(good)
        p[i] = 0
        assert _forward_ex(d, o, 2, p) == glm.EINVAL
    _, need = _ws_ex((64, 128, 8, 64, 64), 2, o)
    assert _forward_ex(d, o, 2, good, FAKE, need - 1) == glm.EWORKSPACE
    assert _forward_ex(d, Options(3, 1, 2, None, 0.0, 0), 2, good, FAKE, need) == glm.EINVAL
    assert _forward_ex(Dims(0, 128, 8, 64, 64, glm.BF16, glm.BF16), o, 2, [0] * 10) == glm.OK


def test_route_ex_checks_options():
    L = glm.lib()
    d = Dims(64, 128, 8, 64, 64, glm.BF16, glm.BF16)
    bad = Options(8, 9, 2, None, 0.0, 0)
    assert L.glm_moe_route_ex(ctypes.byref(d), ctypes.byref(bad), FAKE, FAKE, FAKE, 2, 1.0, FAKE,
                              FAKE, FAKE, 1 << 30, None) == glm.EINVAL


def _dense_ws(T, D, Fs, opts=None, dt=glm.BF16, E=0, F=0):
    n = ctypes.c_size_t(0)
    st = glm.lib().glm_moe_dense_workspace_size(ctypes.byref(Dims(T, D, E, F, Fs, dt, dt)),
                                                opts and ctypes.byref(opts), ctypes.byref(n))
    return st, n.value


def test_dense_workspace():
    st, n = _dense_ws(4096, 6144, 12288)
    assert st == glm.OK
    # hidden activations [T][F] bf16 and the fp32 output staging [T][D]
    assert n >= 4096 * 12288 * 2 + 4096 * 6144 * 4
    # E and F are ignored; grouping options too
    assert _dense_ws(4096, 6144, 12288, E=7, F=3) == (glm.OK, n)
    assert _dense_ws(4096, 6144, 12288, Options(3, 9, 99, None, 0.0, 1)) == (glm.OK, n)
    assert _dense_ws(0, 6144, 12288) == (glm.OK, 0)
    assert _dense_ws(64, 6144, 100)[0] == glm.EUNSUPPORTED
    assert _dense_ws(64, 6144, 0)[0] == glm.EINVAL
    assert _dense_ws(64, 6144, 100, dt=glm.F32)[0] == glm.OK


def test_dense_argument_checks():
    L = glm.lib()
    d = Dims(64, 128, 0, 0, 64, glm.BF16, glm.BF16)
    _, need = _dense_ws(64, 128, 64)
    good = [FAKE] * 5
    for i in range(5):
        p = list(good)
        p[i] = 0
        assert L.glm_moe_dense_ffn(ctypes.byref(d), None, *p, FAKE, need, None,
                                   None) == glm.EINVAL
        p[i] = FAKE + 2
        assert L.glm_moe_dense_ffn(ctypes.byref(d), None, *p, FAKE, need, None,
                                   None) == glm.EINVAL
    assert L.glm_moe_dense_ffn(ctypes.byref(d), None, *good, FAKE, need - 1, None,
                               None) == glm.EWORKSPACE
    d0 = Dims(0, 128, 0, 0, 64, glm.BF16, glm.BF16)
    assert L.glm_moe_dense_ffn(ctypes.byref(d0), None, 0, 0, 0, 0, 0, 0, 0, None,
                               None) == glm.OK


# ----------------------------------------------------------- MXFP8 weights

from sparse_moe_transformer_glm_amd._lib import MxWeights  # noqa: E402


def _mx_dims(T=64, D=6144, E=256, F=2048, Fs=2048):
    return Dims(T, D, E, F, Fs, glm.BF16, glm.MXFP8)


def test_mx_workspace_and_shape_rules():
    n = ctypes.c_size_t(0)
    L = glm.lib()
    assert L.glm_moe_workspace_size_ex(ctypes.byref(_mx_dims()), None, 8, ctypes.byref(n)) == glm.OK
    # hidden rows as 1-byte codes plus a scale per 32: smaller than bf16 hidden rows
    _, nb = _ws(64, 6144, 256, 2048, 2048, 8)
    assert 0 < n.value < nb
    for bad in (_mx_dims(D=6144 + 64), _mx_dims(F=2048 + 64), _mx_dims(Fs=2048 + 64)):
        assert L.glm_moe_workspace_size_ex(ctypes.byref(bad), None, 8,
                                           ctypes.byref(n)) == glm.EUNSUPPORTED
    f32mx = Dims(64, 6144, 256, 2048, 2048, glm.F32, glm.MXFP8)
    assert L.glm_moe_workspace_size_ex(ctypes.byref(f32mx), None, 8,
                                       ctypes.byref(n)) == glm.EUNSUPPORTED
    dense = Dims(64, 6144, 0, 0, 2048, glm.BF16, glm.MXFP8)
    assert L.glm_moe_dense_workspace_size(ctypes.byref(dense), None,
                                          ctypes.byref(n)) == glm.EUNSUPPORTED


def _forward_mx(d, W, ws=FAKE, ws_bytes=1 << 40, k=8, x=FAKE, out=FAKE):
    return glm.lib().glm_moe_forward_mx(ctypes.byref(d), None, x, FAKE, FAKE,
                                        None if W is None else ctypes.byref(W), k, 2.5, out,
                                        None, None, ws, ws_bytes, None, None)


def test_forward_mx_argument_checks():
    d = _mx_dims()
    names = [f for f, _ in MxWeights._fields_]
    good = MxWeights(*([FAKE] * len(names)))
    assert _forward_mx(d, None) == glm.EINVAL
    for i in range(len(names)):
        vals = [FAKE] * len(names)
        vals[i] = 0
        assert _forward_mx(d, MxWeights(*vals)) == glm.EINVAL, names[i]
        vals[i] = FAKE + 4
        assert _forward_mx(d, MxWeights(*vals)) == glm.EINVAL, names[i]
    assert _forward_mx(d, good, x=0) == glm.EINVAL
    assert _forward_mx(d, good, out=0) == glm.EINVAL
    n = ctypes.c_size_t(0)
    glm.lib().glm_moe_workspace_size_ex(ctypes.byref(d), None, 8, ctypes.byref(n))
    assert _forward_mx(d, good, ws_bytes=n.value - 1) == glm.EWORKSPACE
    # bf16 weights through the MXFP8 entry, MXFP8 weights through the bf16 one
    bf = Dims(64, 6144, 256, 2048, 2048, glm.BF16, glm.BF16)
    assert _forward_mx(bf, good) == glm.EINVAL
    ptrs = [FAKE] * 10
    assert glm.lib().glm_moe_forward(ctypes.byref(d), *ptrs[:9], 8, 2.5, ptrs[9], None, None,
                                     FAKE, 1 << 40, None) == glm.EINVAL
    # zero tokens: no-op
    assert _forward_mx(_mx_dims(T=0), None, x=0, out=0) == glm.OK


def test_mx_pack_scales_argument_checks():
    pack = glm.lib().glm_moe_mx_pack_scales
    other = FAKE + (1 << 30)
    assert pack(FAKE, other, 2, 64, 100, None) == glm.EINVAL          # K not a multiple of 128
    assert pack(FAKE, other, 2, 0, 128, None) == glm.EINVAL           # no rows
    assert pack(FAKE, other, -1, 64, 128, None) == glm.EINVAL
    assert pack(0, other, 2, 64, 128, None) == glm.EINVAL             # null source
    assert pack(FAKE, 0, 2, 64, 128, None) == glm.EINVAL
    assert pack(FAKE + 4, other, 2, 64, 128, None) == glm.EINVAL      # misaligned
    assert pack(FAKE, FAKE + 16, 2, 64, 128, None) == glm.EINVAL      # overlapping
    assert pack(0, 0, 0, 64, 128, None) == glm.OK                     # nothing to do
