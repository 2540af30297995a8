"""The C-ABI library without a GPU: it loads, exports every function that
include/swiglu_q.h declares, and rejects bad arguments before any HIP call."""
import os
import re
import subprocess

import pytest

import quantized_swiglu_forward_amd as swq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swiglu_q.h")

# fake, 256-byte aligned "device" addresses: validation never dereferences them
P = 1 << 20


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(swiglu_q_\w+)\s*\(", text)))


def _exported():
    out = subprocess.run(["nm", "-D", "--defined-only", swq.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    return {line.split()[-1] for line in out.splitlines() if " T " in line}


def test_library_exports_every_declared_function():
    declared = _declared_functions()
    assert "swiglu_q_forward" in declared and len(declared) >= 10
    missing = [f for f in declared if f not in _exported()]
    assert not missing, missing
    for f in declared:
        assert hasattr(swq.lib(), f)
        assert hasattr(swq, f), f"binding lacks {f}"


def _fwd(**kw):
    a = dict(x=P, Wg=P, sg=P, bg=P, Wu=P, su=P, bu=P, M=4, H=256, I=64, bits_g=4, gs_g=64, bits_u=4,
             gs_u=64, precision_mode=0, out=P, stream=0)
    a.update(kw)
    return swq.swiglu_q_forward(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), swq.SWQ_ERR_NULL),
    (dict(Wg=None), swq.SWQ_ERR_NULL),
    (dict(bu=None), swq.SWQ_ERR_NULL),
    (dict(out=None), swq.SWQ_ERR_NULL),
    (dict(bits_g=3), swq.SWQ_ERR_UNSUPPORTED),
    (dict(bits_u=6), swq.SWQ_ERR_UNSUPPORTED),
    (dict(bits_g=16), swq.SWQ_ERR_UNSUPPORTED),
    (dict(gs_g=16), swq.SWQ_ERR_UNSUPPORTED),
    (dict(gs_u=96), swq.SWQ_ERR_UNSUPPORTED),
    (dict(precision_mode=3), swq.SWQ_ERR_UNSUPPORTED),
    (dict(precision_mode=-1), swq.SWQ_ERR_UNSUPPORTED),
    (dict(M=-1), swq.SWQ_ERR_SHAPE),
    (dict(H=0), swq.SWQ_ERR_SHAPE),
    (dict(I=0), swq.SWQ_ERR_SHAPE),
    (dict(H=96, gs_g=64), swq.SWQ_ERR_SHAPE),
    (dict(H=200, gs_g=32, gs_u=32), swq.SWQ_ERR_SHAPE),
    (dict(H=(1 << 20) + 64), swq.SWQ_ERR_SHAPE),
    (dict(M=(1 << 30) + 1), swq.SWQ_ERR_SHAPE),
    (dict(M=1 << 30, I=1 << 30), swq.SWQ_ERR_SHAPE),
    (dict(M=1 << 20, H=2048), swq.SWQ_ERR_SHAPE),
    (dict(x=P + 8), swq.SWQ_ERR_ALIGN),
    (dict(Wg=P + 4), swq.SWQ_ERR_ALIGN),
    (dict(Wu=P + 2), swq.SWQ_ERR_ALIGN),
    (dict(sg=P + 1), swq.SWQ_ERR_ALIGN),
    (dict(out=P + 1), swq.SWQ_ERR_ALIGN),
    (dict(out=P + 2, precision_mode=1), swq.SWQ_ERR_ALIGN),
])
def test_forward_validation(kw, status):
    before = (swq.swiglu_q_call_count(0), swq.swiglu_q_call_count(1))
    assert _fwd(**kw) == status
    assert (swq.swiglu_q_call_count(0), swq.swiglu_q_call_count(1)) == before


def test_m_zero_is_ok_and_launches_nothing():
    before = (swq.swiglu_q_call_count(0), swq.swiglu_q_call_count(1))
    assert _fwd(M=0) == swq.SWQ_OK
    assert (swq.swiglu_q_call_count(0), swq.swiglu_q_call_count(1)) == before


def test_debug_gemm_validation():
    base = dict(x=P, Wg=P, sg=P, bg=P, Wu=P, su=P, bu=P, M=4, H=256, I=64, bits_g=4, gs_g=64,
                bits_u=4, gs_u=64, path=-1, gate_out=P, up_out=P, stream=0)
    assert swq.swiglu_q_debug_gemm(**{**base, "path": 2}) == swq.SWQ_ERR_UNSUPPORTED
    assert swq.swiglu_q_debug_gemm(**{**base, "gate_out": None}) == swq.SWQ_ERR_NULL
    assert swq.swiglu_q_debug_gemm(**{**base, "up_out": P + 2}) == swq.SWQ_ERR_ALIGN
    assert swq.swiglu_q_debug_gemm(**{**base, "bits_g": 5}) == swq.SWQ_ERR_UNSUPPORTED
    assert swq.swiglu_q_debug_gemm(**{**base, "M": 0}) == swq.SWQ_OK
    # the matrix-vector path cannot take this many rows
    assert swq.swiglu_q_debug_gemm(**{**base, "M": 4096, "path": 0}) == swq.SWQ_ERR_UNSUPPORTED


def test_linear_validation():
    """swiglu_q_linear checks its arguments before any HIP call: M = 0 is a
    no-op, bad shapes, specs, output types and alignments are rejected."""
    base = dict(x=P, W=P, s=P, b=P, M=4, K=256, N=65, bits=4, gs=64, out_mode=0, out=P, stream=0)
    before = (swq.swiglu_q_call_count(0), swq.swiglu_q_call_count(1))
    assert swq.swiglu_q_linear(**{**base, "M": 0}) == swq.SWQ_OK
    assert swq.swiglu_q_linear(**{**base, "W": None}) == swq.SWQ_ERR_NULL
    assert swq.swiglu_q_linear(**{**base, "out": None}) == swq.SWQ_ERR_NULL
    assert swq.swiglu_q_linear(**{**base, "N": 0}) == swq.SWQ_ERR_SHAPE
    assert swq.swiglu_q_linear(**{**base, "N": -3}) == swq.SWQ_ERR_SHAPE
    assert swq.swiglu_q_linear(**{**base, "K": 96}) == swq.SWQ_ERR_SHAPE        # not a multiple of gs
    assert swq.swiglu_q_linear(**{**base, "K": 80, "gs": 32}) == swq.SWQ_ERR_SHAPE
    assert swq.swiglu_q_linear(**{**base, "M": -1}) == swq.SWQ_ERR_SHAPE
    assert swq.swiglu_q_linear(**{**base, "bits": 3}) == swq.SWQ_ERR_UNSUPPORTED
    assert swq.swiglu_q_linear(**{**base, "gs": 16}) == swq.SWQ_ERR_UNSUPPORTED
    assert swq.swiglu_q_linear(**{**base, "out_mode": 2}) == swq.SWQ_ERR_UNSUPPORTED
    assert swq.swiglu_q_linear(**{**base, "x": P + 8}) == swq.SWQ_ERR_ALIGN
    assert swq.swiglu_q_linear(**{**base, "W": P + 4}) == swq.SWQ_ERR_ALIGN
    assert swq.swiglu_q_linear(**{**base, "s": P + 1}) == swq.SWQ_ERR_ALIGN
    assert swq.swiglu_q_linear(**{**base, "out": P + 1}) == swq.SWQ_ERR_ALIGN
    assert swq.swiglu_q_linear(**{**base, "out": P + 2, "out_mode": 1}) == swq.SWQ_ERR_ALIGN
    assert (swq.swiglu_q_call_count(0), swq.swiglu_q_call_count(1)) == before


def test_mlp_validation():
    """swiglu_q_mlp checks the forward's and the down projection's arguments
    before any HIP call (the hidden buffer included): M = 0 is a no-op; bad
    shapes, specs, output types and alignments are rejected."""
    base = dict(x=P, Wg=P, sg=P, bg=P, Wu=P, su=P, bu=P, Wd=P, sd=P, bd=P, residual=P, M=4, H=256, I=512,
                Ho=256, bits_g=4, gs_g=64, bits_u=4, gs_u=64, bits_d=4, gs_d=64, out_mode=0, out=P, stream=0)
    before = (swq.swiglu_q_call_count(0), swq.swiglu_q_call_count(1))
    assert swq.swiglu_q_mlp(**{**base, "M": 0}) == swq.SWQ_OK
    assert swq.swiglu_q_mlp(**{**base, "M": 0, "residual": None}) == swq.SWQ_OK
    assert swq.swiglu_q_mlp(**{**base, "x": None}) == swq.SWQ_ERR_NULL
    assert swq.swiglu_q_mlp(**{**base, "Wd": None}) == swq.SWQ_ERR_NULL
    assert swq.swiglu_q_mlp(**{**base, "bd": None}) == swq.SWQ_ERR_NULL
    assert swq.swiglu_q_mlp(**{**base, "out": None}) == swq.SWQ_ERR_NULL
    assert swq.swiglu_q_mlp(**{**base, "bits_d": 3}) == swq.SWQ_ERR_UNSUPPORTED
    assert swq.swiglu_q_mlp(**{**base, "gs_d": 16}) == swq.SWQ_ERR_UNSUPPORTED
    assert swq.swiglu_q_mlp(**{**base, "bits_g": 5}) == swq.SWQ_ERR_UNSUPPORTED
    assert swq.swiglu_q_mlp(**{**base, "out_mode": 2}) == swq.SWQ_ERR_UNSUPPORTED
    assert swq.swiglu_q_mlp(**{**base, "I": 480}) == swq.SWQ_ERR_SHAPE          # down: I not a multiple of gs_d
    assert swq.swiglu_q_mlp(**{**base, "Ho": 0}) == swq.SWQ_ERR_SHAPE
    assert swq.swiglu_q_mlp(**{**base, "H": 96}) == swq.SWQ_ERR_SHAPE
    assert swq.swiglu_q_mlp(**{**base, "I": 1 << 21}) == swq.SWQ_ERR_SHAPE      # the down projection's K limit
    assert swq.swiglu_q_mlp(**{**base, "x": P + 8}) == swq.SWQ_ERR_ALIGN
    assert swq.swiglu_q_mlp(**{**base, "Wd": P + 4}) == swq.SWQ_ERR_ALIGN
    assert swq.swiglu_q_mlp(**{**base, "sd": P + 1}) == swq.SWQ_ERR_ALIGN
    assert swq.swiglu_q_mlp(**{**base, "residual": P + 1}) == swq.SWQ_ERR_ALIGN
    assert swq.swiglu_q_mlp(**{**base, "out": P + 2, "out_mode": 1}) == swq.SWQ_ERR_ALIGN
    assert (swq.swiglu_q_call_count(0), swq.swiglu_q_call_count(1)) == before


def test_header_compiles_as_c_and_links(tmp_path):
    """A plain C99 program includes include/swiglu_q.h, links the library and
    gets the documented status codes from the host-side validation."""
    import shutil
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path / "c_abi_check")
    src = os.path.join(ROOT, "tests", "c_abi_check.c")
    libdir = os.path.dirname(swq.LIB_PATH)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), src,
                    "-L", libdir, "-lswiglu_q", f"-Wl,-rpath,{libdir}", "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert "c abi ok" in r.stdout


def test_supported_predicate():
    assert swq.swiglu_q_supported(2048, 4, 64, 4, 64, 0) == 1
    assert swq.swiglu_q_supported(2560, 8, 32, 4, 64, 1) == 1
    assert swq.swiglu_q_supported(4096, 4, 128, 8, 128, 2) == 1
    assert swq.swiglu_q_supported(2048, 2, 64, 4, 64, 0) == 1
    assert swq.swiglu_q_supported(2048, 3, 64, 4, 64, 0) == 0
    assert swq.swiglu_q_supported(2048, 4, 64, 6, 64, 0) == 0
    assert swq.swiglu_q_supported(2048, 4, 48, 4, 64, 0) == 0
    assert swq.swiglu_q_supported(96, 4, 64, 4, 32, 0) == 0
    assert swq.swiglu_q_supported(2048, 4, 64, 4, 64, 7) == 0


def test_threshold_roundtrip():
    try:
        swq.swiglu_q_set_m_threshold(9)
        assert swq.swiglu_q_get_m_threshold() == 9
        swq.swiglu_q_set_m_threshold(0)
        assert swq.swiglu_q_get_m_threshold() == 0
        swq.swiglu_q_set_m_threshold(-5)   # back to the default rule
        assert swq.swiglu_q_get_m_threshold() == 65
    finally:
        swq.swiglu_q_set_m_threshold(-1)


def test_default_rule_by_weight_size():
    """Without a threshold set, M < 65 takes the matrix-vector path, or
    M < 33 for wide weights (H * I >= 3 * 2^23 with I >= 4096); a threshold
    set by API applies to every shape."""
    swq.swiglu_q_set_m_threshold(-1)
    try:
        for M in (1, 17, 32, 33, 48, 64):
            assert swq.swiglu_q_path_for(M, 2048, 5632) == swq.SWQ_PATH_GEMV, M
            assert swq.swiglu_q_path_for(M, 2048, 8192) == swq.SWQ_PATH_GEMV, M    # 2^24
            assert swq.swiglu_q_path_for(M, 2048, 12287) == swq.SWQ_PATH_GEMV, M   # just below 3 * 2^23
            assert swq.swiglu_q_path_for(M, 14336, 2048) == swq.SWQ_PATH_GEMV, M   # 2048 columns
        for M in (65, 128, 129):
            assert swq.swiglu_q_path_for(M, 2048, 5632) == swq.SWQ_PATH_MFMA, M
        for M in (1, 16, 32):
            assert swq.swiglu_q_path_for(M, 4096, 14336) == swq.SWQ_PATH_GEMV, M
            assert swq.swiglu_q_path_for(M, 2048, 12288) == swq.SWQ_PATH_GEMV, M
        for M in (33, 48, 64, 128):
            assert swq.swiglu_q_path_for(M, 4096, 14336) == swq.SWQ_PATH_MFMA, M
            assert swq.swiglu_q_path_for(M, 2048, 12288) == swq.SWQ_PATH_MFMA, M   # 3 * 2^23
            assert swq.swiglu_q_path_for(M, 6144, 4096) == swq.SWQ_PATH_MFMA, M
        # small weights (H * I <= 2^23): the matrix-vector path up to 128 rows
        for M in (65, 100, 128):
            assert swq.swiglu_q_path_for(M, 1024, 4096) == swq.SWQ_PATH_GEMV, M
            assert swq.swiglu_q_path_for(M, 2048, 4096) == swq.SWQ_PATH_GEMV, M   # exactly 2^23
            assert swq.swiglu_q_path_for(M, 2048, 4097) == swq.SWQ_PATH_MFMA, M
        assert swq.swiglu_q_path_for(129, 1024, 4096) == swq.SWQ_PATH_MFMA
        swq.swiglu_q_set_m_threshold(65)
        assert swq.swiglu_q_path_for(64, 4096, 14336) == swq.SWQ_PATH_GEMV
        assert swq.swiglu_q_path_for(65, 1024, 4096) == swq.SWQ_PATH_MFMA
    finally:
        swq.swiglu_q_set_m_threshold(-1)


def test_dispatcher_choice_given_m_and_threshold():
    """M < T takes the matrix-vector path while it fits (M <= 128, row groups
    of 32 past 32 rows), else the MFMA path; T <= 1 sends everything to
    MFMA; invalid sizes give -1."""
    try:
        swq.swiglu_q_set_m_threshold(33)
        for M in (1, 2, 4, 5, 16, 17, 32):
            assert swq.swiglu_q_path_for(M, 2048, 5632) == swq.SWQ_PATH_GEMV, M
        for M in (33, 64, 2048):
            assert swq.swiglu_q_path_for(M, 2048, 5632) == swq.SWQ_PATH_MFMA, M
        swq.swiglu_q_set_m_threshold(9)
        assert swq.swiglu_q_path_for(8, 4096, 14336) == swq.SWQ_PATH_GEMV
        assert swq.swiglu_q_path_for(9, 4096, 14336) == swq.SWQ_PATH_MFMA
        swq.swiglu_q_set_m_threshold(200)
        assert swq.swiglu_q_path_for(32, 256, 768) == swq.SWQ_PATH_GEMV
        assert swq.swiglu_q_path_for(128, 256, 768) == swq.SWQ_PATH_GEMV  # four row groups of 32
        assert swq.swiglu_q_path_for(129, 256, 768) == swq.SWQ_PATH_MFMA   # past the matrix-vector limit
        swq.swiglu_q_set_m_threshold(1)
        assert swq.swiglu_q_path_for(1, 2048, 5632) == swq.SWQ_PATH_MFMA
        assert swq.swiglu_q_path_for(0, 2048, 5632) == -1 and swq.swiglu_q_path_for(4, 0, 5632) == -1
        assert swq.swiglu_q_path_for(4, 2048, 0) == -1
    finally:
        swq.swiglu_q_set_m_threshold(-1)


def test_threshold_default_from_environment():
    code = ("import quantized_swiglu_forward_amd as s; print(s.swiglu_q_get_m_threshold())")
    env = dict(os.environ, SWIGLU_Q_MMIN="13")
    out = subprocess.run(["python", "-c", code], capture_output=True, text=True, env=env, cwd=ROOT,
                         check=True).stdout.strip()
    assert out == "13"
    env = dict(os.environ, SWIGLU_Q_MMIN="junk")
    out = subprocess.run(["python", "-c", code], capture_output=True, text=True, env=env, cwd=ROOT,
                         check=True).stdout.strip()
    assert out == "65"


def test_strerror_and_version():
    for s in range(7):
        assert swq.swiglu_q_strerror(s)
    assert swq.swiglu_q_strerror(99) == "unknown status"
    assert "gfx950" in swq.swiglu_q_version()


def test_workspace_bytes():
    # x' rows of H + extra columns (3 per group of the finer group size,
    # padded to 32) halves, row exponents, one [I, kext] binary16 plane of
    # extra-column B rows per matrix, 4 KB of scale tile per 128 columns and
    # 128 inputs, then the weight rows' exponents (int32, gate and up)
    def a256(v):
        return (v + 255) // 256 * 256

    def expect(M, H, I, bg, gg, bu, gu):
        ext = (3 * (H // min(gg, gu)) + 31) // 32 * 32
        tiles = (I + 127) // 128 * ((H + 127) // 128)
        return (a256(M * (H + ext) * 2) + a256(M * 4) + 2 * a256(I * ext * 2) + a256(tiles * 4096)
                + a256(2 * I * 4))

    assert swq.swiglu_q_workspace_bytes(512, 2048, 8192, 4, 64, 4, 64) == expect(512, 2048, 8192, 4, 64, 4, 64)
    assert swq.swiglu_q_workspace_bytes(8192, 2560, 10240, 8, 32, 4, 64) == expect(8192, 2560, 10240, 8, 32, 4, 64)
    assert swq.swiglu_q_workspace_bytes(0, 2048, 64, 4, 64, 4, 64) == 0
    assert swq.swiglu_q_workspace_bytes(4, 2048, 64, 3, 64, 4, 64) == 0


def test_workspace_bytes_k_split(monkeypatch):
    # few 128 x 128 tiles (at most half of 256 CUs) and H >= 2048: the K
    # split's float32 partial sums (gate and up, [splits, M, I]) follow,
    # min(256 / tiles, K-steps / 16, 8 or from 256 K-steps 16) splits, more
    # than two only below 32 MB
    def a256(v):
        return (v + 255) // 256 * 256

    def base(M, H, I):
        ext = (3 * (H // 64) + 31) // 32 * 32
        tiles = (I + 127) // 128 * ((H + 127) // 128)
        return a256(M * (H + ext) * 2) + a256(M * 4) + 2 * a256(I * ext * 2) + a256(tiles * 4096) + a256(2 * I * 4)

    ws = lambda M, H, I: swq.swiglu_q_workspace_bytes(M, H, I, 4, 64, 4, 64)
    monkeypatch.delenv("SWIGLU_Q_MFMA_KSPLIT", raising=False)
    # 44 tiles, 64 K-steps: four splits
    assert ws(65, 2048, 5632) == base(65, 2048, 5632) + a256(2 * 4 * 65 * 5632 * 4)
    # 64 tiles, 128 K-steps: four splits (32 MiB of partial sums) lower to three
    assert ws(128, 4096, 8192) == base(128, 4096, 8192) + a256(2 * 3 * 128 * 8192 * 4)
    # 3 tiles at H = 4096: eight splits; 16 tiles at H = 14336 (448 K-steps): sixteen
    assert ws(96, 4096, 384) == base(96, 4096, 384) + a256(2 * 8 * 96 * 384 * 4)
    assert ws(48, 14336, 2048) == base(48, 14336, 2048) + a256(2 * 16 * 48 * 2048 * 4)
    # H = 1024 (32 K-steps) and 2 x 112 tiles: none
    assert ws(65, 1024, 4096) == base(65, 1024, 4096)
    assert ws(256, 4096, 14336) == base(256, 4096, 14336)
    # 112 tiles: two splits (29.4 MB); 128 tiles: two splits (32 MiB)
    assert ws(256, 4096, 8192) == base(256, 4096, 8192) + a256(2 * 2 * 256 * 8192 * 4)
    assert ws(128, 4096, 14336) == base(128, 4096, 14336) + a256(2 * 2 * 128 * 14336 * 4)
    # capped by the environment: three, then none
    monkeypatch.setenv("SWIGLU_Q_MFMA_KSPLIT", "3")
    assert ws(96, 4096, 384) == base(96, 4096, 384) + a256(2 * 3 * 96 * 384 * 4)
    monkeypatch.setenv("SWIGLU_Q_MFMA_KSPLIT", "0")
    assert ws(96, 4096, 384) == base(96, 4096, 384)


def test_few_row_x_source_and_workspace():
    """The few-row kernel converts x itself (no prep launch, no workspace)
    for M <= 16 when a row fits one pass of its waves and their LDS regions
    (skinny_self_region each) fit 64 KB: up to H = 4096 with equal code
    widths of at most 4 bits (two chunk quads per wave; M <= 8 there), up to
    H = 2048 otherwise; for 16 < M <= 32 (two row tiles) with equal code
    widths of at most 4 bits and one chunk quad per wave, up to H = 2048
    (8 KB regions within 128 KB); other calls take x' from the prep kernel,
    and SWIGLU_Q_SKINNY_X=prep forces that."""
    def ws(M, H, bg=4, bu=4):
        return swq.swiglu_q_staging_bytes(M, H, 5632, bg, 64, bu, 64)

    def prep_bytes(M, H):   # x' in lane order, row exponents, weight-row exponents
        a = lambda v: (v + 255) // 256 * 256
        tiles = 2 * ((M + 31) // 32) if M > 16 else 1   # 16-row tiles: two per row group of 32
        return a((H + 127) // 128 * tiles * 256 * 16) + a(M * 4) + a(2 * 5632 * 4)

    for M, H in ((5, 2048), (8, 2048), (16, 2048), (8, 4096), (2, 1024), (16, 1056)):
        assert ws(M, H) == 0, (M, H)
    assert ws(16, 2048, 8, 8) == 0 and ws(8, 2048, 4, 8) == 0
    assert ws(9, 4096) == prep_bytes(9, 4096)     # 16 waves x 8 KB of LDS
    assert ws(8, 4096, 8, 8) == prep_bytes(8, 4096)
    assert ws(17, 2048) == 0 and ws(32, 1024) == 0 and ws(32, 2048, 2, 2) == 0 and ws(24, 512) == 0
    assert ws(17, 2048, 8, 4) == prep_bytes(17, 2048)   # codes not narrow
    assert ws(24, 4096) == prep_bytes(24, 4096)         # 32 quads: no one pass of one quad per wave
    # row groups of 32 past 32 rows: converted by the waves, or staged for every group
    gemv = lambda M, H: swq.swiglu_q_staging_bytes(M, H, 5632, 4, 64, 4, 64, swq.SWQ_PATH_GEMV)
    assert ws(33, 2048) == 0 and ws(64, 2048, 2, 2) == 0 and gemv(128, 1024) == 0
    assert ws(40, 2048, 8, 4) == prep_bytes(40, 2048) and gemv(128, 4096) == prep_bytes(128, 4096)
    assert ws(8, 8192) == prep_bytes(8, 8192)
    os.environ["SWIGLU_Q_SKINNY_X"] = "prep"
    try:
        assert ws(8, 2048) == prep_bytes(8, 2048)
    finally:
        os.environ.pop("SWIGLU_Q_SKINNY_X")
    assert ws(8, 2048) == 0
    # M = 1 reads x itself; the matrix-matrix path stages its workspace
    assert ws(1, 2048) == 0
    assert swq.swiglu_q_staging_bytes(512, 2048, 8192, 4, 64, 4, 64) == \
        swq.swiglu_q_workspace_bytes(512, 2048, 8192, 4, 64, 4, 64)
    assert swq.swiglu_q_staging_bytes(8, 2048, 5632, 4, 64, 4, 64, swq.SWQ_PATH_MFMA) == \
        swq.swiglu_q_workspace_bytes(8, 2048, 5632, 4, 64, 4, 64)
    assert swq.swiglu_q_staging_bytes(129, 2048, 5632, 4, 64, 4, 64, swq.SWQ_PATH_GEMV) == 0   # no such call
    assert swq.swiglu_q_staging_bytes(8, 2048, 5632, 3, 64, 4, 64) == 0


def test_binding_has_no_fallback():
    """The binding only marshals: it never imports the oracle."""
    src = open(os.path.join(ROOT, "quantized_swiglu_forward_amd", "__init__.py")).read()
    assert "oracle" not in src


def test_tensor_helpers_reject_other_activation_types():
    """The tensor conveniences take bf16 activations (or their 16-bit bit
    patterns) only: a float16 or float32 x is refused before any call into
    the library, instead of being read as bf16 bits."""
    import torch
    w = torch.zeros((64, 32), dtype=torch.int32)
    s = torch.zeros((64, 4), dtype=torch.bfloat16)
    for dt in (torch.float16, torch.float32):
        x = torch.zeros((2, 256), dtype=dt)
        with pytest.raises(TypeError):
            swq.forward(x, w, s, s, w, s, s, 4, 64)
        with pytest.raises(TypeError):
            swq.linear(x, w, s, s, 4, 64)
        with pytest.raises(TypeError):
            swq.debug_gemm_tensors(x, w, s, s, w, s, s, 4, 64)
        with pytest.raises(TypeError):
            swq.mlp(x, w, s, s, w, s, s, w, s, s, (4, 64), (4, 64), (4, 64))


def test_tensor_helpers_collapse_leading_dimensions():
    """x of shape [..., H] becomes M = prod(...) rows of one contiguous block
    (the pages' host entry does the same), and a non-contiguous x is refused."""
    import torch
    x = torch.zeros((2, 3, 5, 256), dtype=torch.bfloat16)
    x2, lead = swq._rows(x, "t")
    assert tuple(x2.shape) == (30, 256) and lead == (2, 3, 5) and x2.data_ptr() == x.data_ptr()
    x2, lead = swq._rows(torch.zeros((256,), dtype=torch.int16), "t")
    assert tuple(x2.shape) == (1, 256) and lead == ()
    with pytest.raises(ValueError):
        swq._rows(torch.zeros((256, 4), dtype=torch.bfloat16).t(), "t")


def test_noalloc_rejects_oversized_calls_before_any_hip_call():
    """The allocation-free forward refuses a call whose staging would exceed
    its fixed 64 MiB with SWQ_ERR_TOO_LARGE, and validates like the forward,
    all on the host (no device is touched: these run without a GPU)."""
    a = dict(x=P, Wg=P, sg=P, bg=P, Wu=P, su=P, bu=P, M=8192, H=4096, I=14336, bits_g=4, gs_g=64, bits_u=4,
             gs_u=64, precision_mode=0, out=P, stream=0)
    assert swq.swiglu_q_workspace_bytes(8192, 4096, 14336, 4, 64, 4, 64) > 64 << 20
    assert swq.swiglu_q_forward_noalloc(**a) == swq.SWQ_ERR_TOO_LARGE
    assert swq.swiglu_q_forward_noalloc(**{**a, "M": 0}) == swq.SWQ_OK
    assert swq.swiglu_q_forward_noalloc(**{**a, "x": None}) == swq.SWQ_ERR_NULL
    assert swq.swiglu_q_forward_noalloc(**{**a, "bits_g": 3}) == swq.SWQ_ERR_UNSUPPORTED
    assert swq.swiglu_q_forward_noalloc(**{**a, "precision_mode": 3}) == swq.SWQ_ERR_UNSUPPORTED
    assert swq.swiglu_q_forward_noalloc(**{**a, "out": P + 1}) == swq.SWQ_ERR_ALIGN
    assert "64 MiB" in swq.swiglu_q_strerror(swq.SWQ_ERR_TOO_LARGE)


def test_call_cap_predicate():
    """The bisecting cap: under_cap is 1 while fewer calls than the cap have
    launched, and always 1 without a cap (host only; the library never
    refuses a call itself)."""
    swq.swiglu_q_reset_counts()
    swq.swiglu_q_set_max_calls(-1)
    assert swq.swiglu_q_under_cap() == 1
    swq.swiglu_q_set_max_calls(0)
    assert swq.swiglu_q_under_cap() == 0
    swq.swiglu_q_set_max_calls(3)
    assert swq.swiglu_q_under_cap() == 1
    swq.swiglu_q_set_max_calls(-5)
    assert swq.swiglu_q_under_cap() == 1


def test_hip_failure_maps_to_err_hip():
    """Without a GPU every HIP call fails; a valid call that reaches HIP (a
    matrix-matrix call needs its workspace, a decode call launches, the
    allocation-free call needs the scratch array's address) returns
    SWQ_ERR_HIP instead of crashing.  Skipped where a GPU is visible: there the
    fake pointers would reach a kernel."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("needs a machine without a GPU")
    base = dict(x=P, Wg=P, sg=P, bg=P, Wu=P, su=P, bu=P, H=256, I=64, bits_g=4, gs_g=64, bits_u=4,
                gs_u=64, precision_mode=0, out=P, stream=0)
    assert swq.swiglu_q_forward(**{**base, "M": 300}) == swq.SWQ_ERR_HIP
    assert swq.swiglu_q_forward(**{**base, "M": 1}) == swq.SWQ_ERR_HIP
    assert swq.swiglu_q_forward_noalloc(**{**base, "M": 300}) == swq.SWQ_ERR_HIP
