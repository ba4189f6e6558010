"""libks host logic without a GPU: the library loads, exports every entry
point include/ks.h declares, and rejects bad arguments with the documented
status before any HIP call (these calls never reach the device)."""
import os
import re
import subprocess

import pytest

from kronecker_sparse_structured_amd import libks

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ks.h")

# Fake, well-aligned device addresses far apart; validation never dereferences.
XP, WP, YP, WSP = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ks_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return libks.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"ks_matmul", "ks_chain_matmul", "ks_chain_workspace_size"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", libks.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (ks_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        getattr(lib, n)


def test_status_strings_and_version():
    for i, name in enumerate(libks.STATUS):
        assert libks.ks_status_string(i).startswith(name)
    assert libks.ks_status_string(999) == "KS_ERR_UNKNOWN"
    assert "gfx950" in libks.ks_version()


def st(p, W=WP, X=XP, Y=YP, batch=4, dtype=libks.DTYPE_F32, **kw):
    return libks.ks_matmul_ex(p, W, X, Y, batch, dtype, stream=0, check=False, **kw)


@pytest.mark.parametrize("p", [(0, 1, 1, 1), (1, 0, 1, 1), (1, 1, -3, 1), (1, 1, 1, 0),
                               (1 << 16, 1, 1 << 15, 1), (2, 1 << 30, 2, 1), (1, 46341, 46341, 1)])
def test_bad_pattern(p):
    assert st(p) == libks.KS_ERR_PATTERN


def test_bad_batch():
    assert st((2, 2, 2, 2), batch=-1) == libks.KS_ERR_BATCH
    assert st((2, 2, 2, 2), batch=1 << 31) == libks.KS_ERR_BATCH


def test_bad_dtype():
    assert st((2, 2, 2, 2), dtype=3) == libks.KS_ERR_DTYPE
    assert st((2, 2, 2, 2), dtype=-1) == libks.KS_ERR_DTYPE


def test_empty_batch_is_noop_even_with_null_pointers():
    assert st((2, 3, 4, 5), W=None, X=None, Y=None, batch=0) == libks.KS_OK
    assert libks.ks_matmul((2, 3, 4, 5), None, None, None, 0, libks.DTYPE_F32, stream=0, check=False) == 0


def test_null_pointers():
    for kw in ({"W": None}, {"X": None}, {"Y": None}):
        assert st((2, 2, 2, 2), **kw) == libks.KS_ERR_NULL


def test_alignment():
    assert st((2, 2, 2, 2), X=XP + 2) == libks.KS_ERR_ALIGN
    assert st((2, 2, 2, 2), Y=YP + 1) == libks.KS_ERR_ALIGN
    assert st((2, 2, 2, 2), W=WP + 3, dtype=libks.DTYPE_BF16) == libks.KS_ERR_ALIGN
    assert st((2, 2, 2, 2), X=XP + 1, dtype=libks.DTYPE_BF16) == libks.KS_ERR_ALIGN
    # bf16 X on a 2-byte boundary and fp32 Y on a 4-byte boundary are fine for
    # validation; the call then proceeds to the device, which is not tested here.


def test_overlap():
    p = (2, 4, 4, 2)  # n_in = n_out = 16, batch 4 -> 256 bytes each
    assert st(p, Y=XP) == libks.KS_ERR_OVERLAP
    assert st(p, Y=XP + 252) == libks.KS_ERR_OVERLAP      # last 4 bytes of X
    assert st(p, Y=WP + 4) == libks.KS_ERR_OVERLAP
    assert st(p, Y=XP - 256 + 4) == libks.KS_ERR_OVERLAP  # Y tail reaches X head


def test_options():
    assert st((2, 2, 2, 2), kernel=99) == libks.KS_ERR_INVALID
    assert st((2, 2, 2, 2), rows_per_block=-1) == libks.KS_ERR_INVALID
    assert st((2, 2, 2, 2), reserved=[1]) == libks.KS_ERR_INVALID
    assert st((2, 2, 2, 2), reserved=[0, 0, 0, 0, 1]) == libks.KS_ERR_INVALID
    assert st((2, 2, 2, 2), store_waves=3) == libks.KS_ERR_INVALID
    assert st((2, 2, 2, 2), store_waves=-1) == libks.KS_ERR_INVALID
    # a forced family that cannot run the pattern is refused on the host
    assert st((2, 3, 5, 2), kernel="valu") == libks.KS_ERR_UNSUPPORTED
    assert st((2, 3, 5, 2), kernel="mfma") == libks.KS_ERR_UNSUPPORTED


def cst(ps, batch=4, dtype=libks.DTYPE_F32, ws=WSP, ws_bytes=1 << 30, flags=0, Ws=None, X=XP, Y=YP, n=None):
    Ws = Ws if Ws is not None else [WP + 0x100000 * i for i in range(len(ps))]
    return libks.ks_chain_matmul(ps, Ws, X, Y, batch, dtype, ws, ws_bytes, flags, stream=0, n=n, check=False)


def test_chain_validation():
    ok = [(1, 4, 2, 4), (4, 2, 2, 2)]
    assert cst(ok, n=0) == libks.KS_ERR_CHAIN_MISMATCH
    assert cst([(1, 4, 2, 4), (4, 2, 3, 2)]) == libks.KS_ERR_CHAIN_MISMATCH
    assert cst(ok, dtype=libks.DTYPE_BF16W) == libks.KS_ERR_DTYPE
    assert cst(ok, flags=7) == libks.KS_ERR_INVALID
    assert cst(ok, batch=-2) == libks.KS_ERR_BATCH
    assert cst([(1, 4, 0, 4)]) == libks.KS_ERR_PATTERN
    assert cst(ok, batch=0, X=None, Y=None, ws=None, ws_bytes=0) == libks.KS_OK
    assert cst(ok, X=None) == libks.KS_ERR_NULL
    assert cst(ok, Ws=[WP, None]) == libks.KS_ERR_NULL
    need = libks.ks_chain_workspace_size(ok, 4, libks.DTYPE_F32, libks.CHAIN_NO_FUSE)
    assert cst(ok, flags=libks.CHAIN_NO_FUSE, ws=None, ws_bytes=need) == libks.KS_ERR_WORKSPACE
    assert cst(ok, flags=libks.CHAIN_NO_FUSE, ws_bytes=need - 1) == libks.KS_ERR_WORKSPACE
    assert cst(ok, flags=libks.CHAIN_NO_FUSE, ws=WSP + 8, ws_bytes=need) == libks.KS_ERR_ALIGN
    assert cst(ok, flags=libks.CHAIN_NO_FUSE, ws=XP, ws_bytes=need) == libks.KS_ERR_OVERLAP
    assert cst(ok, Y=XP) == libks.KS_ERR_OVERLAP
    assert cst(ok, Y=WP + 0x100000) == libks.KS_ERR_OVERLAP
    assert cst(ok, X=XP + 2) == libks.KS_ERR_ALIGN


def test_chain_workspace_sizes():
    f32, nf = libks.DTYPE_F32, libks.CHAIN_NO_FUSE
    assert libks.ks_chain_workspace_size([(2, 3, 4, 5)], 10, f32, nf) == 0
    # two factors: one fp32 intermediate of batch x 16, rounded up to 256 bytes
    two = [(1, 4, 2, 4), (4, 2, 2, 2)]
    assert libks.ks_chain_workspace_size(two, 10, f32, nf) == 768
    assert libks.ks_chain_workspace_size(two, 0, f32, nf) == 0
    # three or more: two ping-pong buffers of the widest intermediate
    three = [(1, 6, 2, 3), (3, 2, 3, 2), (2, 2, 3, 2)]   # 6 -> 18 -> 12 -> 8
    assert libks.ks_chain_workspace_size(three, 100, f32, nf) == 2 * 7424
    # bf16 chains keep fp32 intermediates
    assert libks.ks_chain_workspace_size(two, 10, libks.DTYPE_BF16, nf) == 768
    st_, _ = libks.ks_chain_workspace_size(two, 10, libks.DTYPE_BF16W, nf, check=False)
    assert st_ == libks.KS_ERR_DTYPE


def test_plan_describe():
    assert libks.ks_plan_describe((1, 16, 16, 4096), 4096, libks.DTYPE_F32).startswith("mfma")
    assert "segmented" in libks.ks_plan_describe((1, 16, 16, 4096), 4096, libks.DTYPE_F32)
    assert libks.ks_plan_describe((1, 8, 8, 4096), 4096, libks.DTYPE_F32).startswith("valu lane")
    assert libks.ks_plan_describe((4096, 8, 8, 1), 4096, libks.DTYPE_F32).startswith("valu slab")
    assert "outputs/tile=64 of 128" in libks.ks_plan_describe((1, 128, 128, 32), 4096, libks.DTYPE_F32)
    assert libks.ks_plan_describe((2, 3, 5, 7), 10, libks.DTYPE_F32).startswith("generic")


def test_chain_plan():
    three = [(1, 6, 2, 3), (3, 2, 3, 2), (2, 2, 3, 2)]
    assert libks.ks_chain_plan(three, 10, libks.DTYPE_F32, libks.CHAIN_NO_FUSE) == [1, 1, 1]
    assert libks.ks_chain_groups(three, 10, libks.DTYPE_F32, libks.CHAIN_NO_FUSE) == [[0], [1], [2]]
    # small blocks, rows of at most 4096: the whole chain is one row-resident launch
    assert libks.ks_chain_groups(three, 10, libks.DTYPE_F32, libks.CHAIN_AUTO) == [[0, 1, 2]]


def test_chain_plan_row_resident_runs():
    """Runs of small-block factors (b * c <= 16) whose rows fit on chip
    become one launch; a factor with larger blocks or rows over 4096
    elements ends the run."""
    radix2 = [(2 ** k, 2, 2, 2 ** (11 - k)) for k in range(12)]       # n = 4096
    assert libks.ks_chain_groups(radix2, 100, libks.DTYPE_F32) == [list(range(12))]
    assert libks.ks_chain_groups(radix2, 100, libks.DTYPE_F32, libks.CHAIN_NO_FUSE) == [[k] for k in range(12)]
    wide = [(2 ** k, 2, 2, 2 ** (12 - k)) for k in range(13)]          # n = 8192
    assert libks.ks_chain_groups(wide, 100, libks.DTYPE_F32) == [[k] for k in range(13)]
    mixed = [(64, 4, 4, 4), (1, 64, 16, 64), (256, 4, 4, 4), (256, 4, 4, 4)]
    assert libks.ks_chain_groups(mixed, 100, libks.DTYPE_F32) == [[0], [1], [2, 3]]
    big_blocks = [(1, 16, 8, 256), (16, 2, 2, 128), (32, 2, 2, 64)]    # 16 x 8 blocks first
    for dt in (libks.DTYPE_F32, libks.DTYPE_BF16):
        assert libks.ks_chain_groups(big_blocks, 100, dt) == [[0], [1, 2]]
    assert libks.ks_chain_groups([(16, 8, 8, 8), (128, 8, 8, 1)], 100, libks.DTYPE_F32) == [[0], [1]]


def test_chain_plan_fuses_known_pairs():
    """The planner fuses the GPT-2 pair (rows shared by groups of beta0) and
    the butterfly's last two factors (the second works inside the first's
    output slabs); nothing else in those chains, and nothing with NO_FUSE."""
    gpt2 = [(1, 64, 16, 64), (64, 8, 8, 8)]
    bfly = [(16 ** k, 16, 16, 16 ** (3 - k)) for k in range(4)]
    for dt in (libks.DTYPE_F32, libks.DTYPE_BF16):
        assert libks.ks_chain_groups(gpt2, 1000, dt) == [[0, 1]]
        assert libks.ks_chain_groups(bfly, 1000, dt) == [[0], [1], [2, 3]]
        assert libks.ks_chain_groups(bfly, 1000, dt, libks.CHAIN_NO_FUSE) == [[0], [1], [2], [3]]
    # slab family: (a, 16, 16, 16) -> (16 a, 16, 16, 1) for any a; other shapes stay apart
    assert libks.ks_chain_groups([(3, 16, 16, 16), (48, 16, 16, 1)], 7, libks.DTYPE_F32) == [[0, 1]]
    assert libks.ks_chain_groups([(4, 16, 16, 16), (64, 16, 8, 2)], 7, libks.DTYPE_F32) == [[0], [1]]
    assert libks.ks_chain_groups([(4, 8, 16, 16), (32, 16, 16, 1)], 7, libks.DTYPE_F32) == [[0], [1]]


def test_one_hip_runtime_whatever_the_import_order():
    """Loading libks before torch must still leave a single HIP runtime in
    the process (torch bundles its own; libks has to bind to that one)."""
    import sys
    code = ("from kronecker_sparse_structured_amd import libks; libks.load(); "
            "print(len(libks._hip_runtimes()))")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1"


def test_backward_workspace_sizes():
    p = (4, 64, 16, 6)
    nnz = 4 * 64 * 16 * 6
    assert libks.ks_matmul_dx_workspace_size(p, libks.DTYPE_F32) == (nnz * 4 + 255) // 256 * 256
    assert libks.ks_matmul_dx_workspace_size(p, libks.DTYPE_BF16) == (nnz * 2 + 255) // 256 * 256
    assert libks.ks_matmul_dw_workspace_size(p, 1, libks.DTYPE_F32) == 0
    big = libks.ks_matmul_dw_workspace_size(p, 25216, libks.DTYPE_F32)
    assert big % 256 == 0 and big >= 2 * nnz * 4 and big <= 64 << 20
    assert libks.ks_matmul_dx_workspace_size((0, 1, 1, 1), 0, check=False)[0] == libks.KS_ERR_PATTERN
    assert libks.ks_matmul_dw_workspace_size(p, -1, 0, check=False)[0] == libks.KS_ERR_BATCH
    assert libks.ks_matmul_dw_workspace_size(p, 5, 7, check=False)[0] == libks.KS_ERR_DTYPE


def test_backward_argument_errors():
    p = (2, 4, 8, 2)
    need = libks.ks_matmul_dx_workspace_size(p, libks.DTYPE_F32)
    dx = lambda **kw: libks.ks_matmul_dx(kw.get("p", p), kw.get("W", WP), kw.get("dY", XP), kw.get("dX", YP),
                                         kw.get("batch", 4), kw.get("dt", libks.DTYPE_F32), kw.get("ws", WSP),
                                         kw.get("wsb", need), stream=0, check=False)
    assert dx(p=(1, 0, 1, 1)) == libks.KS_ERR_PATTERN
    assert dx(batch=-2) == libks.KS_ERR_BATCH
    assert dx(dt=9) == libks.KS_ERR_DTYPE
    assert dx(batch=0, W=None, dY=None, dX=None, ws=None) == libks.KS_OK
    assert dx(W=None) == libks.KS_ERR_NULL
    assert dx(ws=None) == libks.KS_ERR_WORKSPACE
    assert dx(wsb=need - 1) == libks.KS_ERR_WORKSPACE
    assert dx(dX=YP + 2) == libks.KS_ERR_ALIGN
    assert dx(ws=WSP + 4) == libks.KS_ERR_ALIGN
    assert dx(dX=XP) == libks.KS_ERR_OVERLAP          # dX over dY
    assert dx(ws=WP) == libks.KS_ERR_OVERLAP          # workspace over W
    dw = lambda **kw: libks.ks_matmul_dw(kw.get("p", p), kw.get("dY", YP), kw.get("X", XP), kw.get("dW", WP),
                                         kw.get("batch", 1), kw.get("dt", libks.DTYPE_F32), kw.get("ws", None),
                                         kw.get("wsb", 0), stream=0, check=False)
    assert libks.ks_matmul_dw_workspace_size(p, 1, libks.DTYPE_F32) == 0    # one row range: no partial sums
    assert dw(p=(1, 1, 1, 0)) == libks.KS_ERR_PATTERN
    assert dw(batch=-1) == libks.KS_ERR_BATCH
    assert dw(dt=5) == libks.KS_ERR_DTYPE
    assert dw(dW=None) == libks.KS_ERR_NULL
    assert dw(X=None) == libks.KS_ERR_NULL
    assert dw(dW=WP + 1) == libks.KS_ERR_ALIGN
    assert dw(dW=XP) == libks.KS_ERR_OVERLAP
    big = (64, 8, 8, 8)
    need_w = libks.ks_matmul_dw_workspace_size(big, 4096, libks.DTYPE_F32)
    assert need_w > 0
    assert dw(p=big, batch=4096, ws=None, wsb=0) == libks.KS_ERR_WORKSPACE
    assert dw(p=big, batch=4096, ws=WSP, wsb=need_w - 1) == libks.KS_ERR_WORKSPACE
