"""The C-ABI library loads without a GPU, exports every function that
include/*.h declares, and its host-side rules agree with the oracle's.

Only calls that return before touching the HIP runtime are made here (size
queries and argument checks that fail); no kernel is launched.
"""

import ctypes
import glob
import os
import re
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DECL = re.compile(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\**\s+\**\s*(moe_\w+)\s*\(", re.M)


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        names |= set(DECL.findall(open(h).read()))
    return names


@pytest.fixture(scope="module")
def lib():
    import combine_moe_dispatch_layout_amd as m
    return m.load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("moe_dispatch_layout", "moe_dispatch", "moe_combine", "moe_dispatch_capacity",
              "moe_dispatch_layout_workspace_size", "moe_status_string", "moe_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    import combine_moe_dispatch_layout_amd as m
    out = subprocess.run(["nm", "-D", "--defined-only", m.library_path()], check=True,
                         capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_library_exports_only_the_c_abi():
    """The shared library's dynamic symbol table holds the moe_* entry points
    and nothing else (the kernels and C++ launchers stay local)."""
    import shutil
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    import combine_moe_dispatch_layout_amd as m
    out = subprocess.run([nm, "-D", "--defined-only", m.library_path()], capture_output=True,
                         text=True, check=True).stdout
    names = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert names, "no exported symbols"
    assert all(n.startswith("moe_") for n in names), sorted(n for n in names
                                                            if not n.startswith("moe_"))
    assert names == declared_functions()


def test_abi_version_and_status_strings(lib):
    assert lib.moe_abi_version() == 2
    for code in range(5):
        assert lib.moe_status_string(code)
    assert b"unknown" in lib.moe_status_string(99)


def test_capacity_matches_oracle(lib):
    rng = np.random.default_rng(0)
    for _ in range(2000):
        e = int(rng.integers(-2, 520))
        k = int(rng.integers(-1, 18))
        bs = int(rng.integers(-2, 100000))
        a = int(rng.choice([0, 1, 2, 3, 64, 128, 1024, 2048]))
        ours = lib.moe_dispatch_capacity(bs, k, e, a)
        if oracle.check_layout_args(bs, k, e, a) == oracle.OK:
            assert ours == oracle.capacity(bs, k, e, a)
        else:
            assert ours == -1


def test_workspace_size(lib):
    assert lib.moe_dispatch_layout_workspace_size(128, 8, 256) == 0  # one workgroup
    big = lib.moe_dispatch_layout_workspace_size(16384, 8, 512)
    assert big >= 32 * 512 * 4  # one histogram row per workgroup
    assert lib.moe_dispatch_layout_workspace_size(4, 9, 8) == 0  # invalid -> 0


def _i(v):
    return ctypes.c_void_p(v)


FAKE = 0x1000  # a non-null, 16-byte aligned address never dereferenced


@pytest.mark.parametrize("bs,k,e,align", [(4, 1, 0, 128), (4, 1, 513, 128), (4, 0, 8, 128),
                                          (4, 9, 8, 128), (4, 17, 64, 128), (4, 2, 8, 3),
                                          (-1, 2, 8, 128), (1 << 28, 16, 512, 128)])
def test_layout_rejects_like_the_oracle(lib, bs, k, e, align):
    assert oracle.check_layout_args(bs, k, e, align) == oracle.ERR_INVALID_ARG
    rc = lib.moe_dispatch_layout(FAKE, bs, k, e, align, FAKE, FAKE, FAKE, None, None, 0, None)
    assert rc == 1


def test_layout_rejects_missing_workspace(lib):
    rc = lib.moe_dispatch_layout(FAKE, 16384, 8, 256, 128, FAKE, FAKE, FAKE, None, None, 0, None)
    assert rc == 2
    rc = lib.moe_dispatch_layout(FAKE, 16384, 8, 256, 128, FAKE, FAKE, FAKE, None, FAKE + 8,
                                 1 << 20, None)  # misaligned workspace
    assert rc == 2


def test_layout_rejects_null_outputs(lib):
    assert lib.moe_dispatch_layout(FAKE, 4, 2, 8, 128, None, FAKE, FAKE, None, None, 0, None) == 1
    assert lib.moe_dispatch_layout(None, 4, 2, 8, 128, FAKE, FAKE, FAKE, None, None, 0, None) == 1


@pytest.mark.parametrize("hidden,dtype,code", [(0, 0, 1), (48, 0, 1), (96, 1, 1), (64, 2, 3),
                                               (65568, 0, 1)])
def test_dispatch_row_rules(lib, hidden, dtype, code):
    if hidden <= 65536:
        assert oracle.check_row_args(hidden, dtype) == code
    rc = lib.moe_dispatch(FAKE, max(hidden, 1), 4, hidden, FAKE, FAKE, FAKE, 2, 8, FAKE,
                          max(hidden, 1), 64, dtype, FAKE, None, None)
    assert rc == code


def test_dispatch_alignment_rules(lib):
    # misaligned x base, stride not a multiple of 16 bytes, stride < hidden
    assert lib.moe_dispatch(FAKE + 2, 64, 4, 64, FAKE, FAKE, FAKE, 2, 8, FAKE, 64, 64, 0,
                            None, None, None) == 1
    assert lib.moe_dispatch(FAKE, 68, 4, 64, FAKE, FAKE, FAKE, 2, 8, FAKE, 64, 64, 0,
                            None, None, None) == 1
    assert lib.moe_dispatch(FAKE, 32, 4, 64, FAKE, FAKE, FAKE, 2, 8, FAKE, 64, 64, 0,
                            None, None, None) == 1
    # fp8 without scales
    assert lib.moe_dispatch(FAKE, 128, 4, 128, FAKE, FAKE, FAKE, 2, 8, FAKE, 128, 64, 1,
                            None, None, None) == 1
    # negative capacity
    assert lib.moe_dispatch(FAKE, 64, 4, 64, FAKE, FAKE, FAKE, 2, 8, FAKE, 64, -1, 0,
                            None, None, None) == 1


def test_combine_rules(lib):
    args = dict(x=FAKE, xs=64, cap=64, ids=FAKE, idx=FAKE, send=FAKE, sc=FAKE, sh=None, ss=0,
                bs=4, h=64, k=2, e=8, out=FAKE)

    def call(**kw):
        a = dict(args, **kw)
        return lib.moe_combine(a["x"], a["xs"], a["cap"], a["ids"], a["idx"], a["send"], a["sc"],
                               a["sh"], a["ss"], a["bs"], a["h"], a["k"], a["e"], a["out"],
                               None, None)

    assert call(h=48) == 1
    assert call(sc=None) == 1
    assert call(out=FAKE + 4) == 1
    assert call(sh=FAKE, ss=32) == 1       # shared stride < hidden
    assert call(sh=FAKE + 2, ss=64) == 1   # misaligned shared
    assert call(k=9) == 1
    assert call(cap=-5) == 1
    assert call(bs=0) == 0                 # empty batch: nothing to launch


def test_combine_fp8_rules(lib):
    def call(x=FAKE, xs=128, cap=64, qs=FAKE, h=128, sh=None, ss=0, out=FAKE, k=2):
        return lib.moe_combine_fp8(x, xs, cap, qs, FAKE, FAKE, FAKE, FAKE, sh, ss, 4, h, k, 8,
                                   out, None, None)

    assert call(h=64, xs=64) == 1          # hidden must be a multiple of 128
    assert call(qs=None) == 1              # scales required
    assert call(qs=FAKE + 2) == 1          # misaligned scales
    assert call(xs=120) == 1               # stride < hidden
    assert call(x=FAKE + 8) == 1           # misaligned codes
    assert call(sh=FAKE, ss=64) == 1       # shared stride < hidden
    assert call(k=17) == 1
    assert lib.moe_combine_fp8(FAKE, 128, 64, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 0, 128, 2,
                               8, FAKE, None, None) == 0   # empty batch


@pytest.mark.parametrize("e,ws", [(16, 3), (16, 0), (8, 16), (16, -2)])
def test_layout_ep_rejects_like_the_oracle(lib, e, ws):
    with pytest.raises(oracle.OracleArgError):
        oracle.layout_ep(np.zeros((2, 1), np.int32), e, ws, 128)
    assert lib.moe_dispatch_layout_ep(FAKE, 2, 1, e, ws, 128, FAKE, FAKE, FAKE, FAKE, None, None,
                                      0, None) == 1


def test_layout_replicated_rules(lib):
    # replicas must admit k distinct choices; tables are required
    assert lib.moe_dispatch_layout_replicated(FAKE, 4, 2, 8, FAKE, FAKE, 1, 0, 128, FAKE, FAKE,
                                              FAKE, FAKE, None, None, 0, None) == 1
    assert lib.moe_dispatch_layout_replicated(FAKE, 4, 2, 8, None, FAKE, 8, 0, 128, FAKE, FAKE,
                                              FAKE, FAKE, None, None, 0, None) == 1
    assert lib.moe_dispatch_layout_replicated(FAKE, 4, 2, 8, FAKE, FAKE, 513, 0, 128, FAKE,
                                              FAKE, FAKE, FAKE, None, None, 0, None) == 1


def test_dispatch_fused_replicated_rules(lib):
    def call(k=2, e=8, reps=8, hidden=128, dtype=0, offsets=FAKE, thresholds=FAKE,
             cap=64, expand_x=FAKE, scales=None, bs=4):
        return lib.moe_dispatch_fused_replicated(
            FAKE, hidden, bs, hidden, FAKE, k, e, offsets, thresholds, reps, 0, 128, FAKE, FAKE,
            FAKE, FAKE, expand_x, hidden, cap, dtype, scales, None, None, 0, None)

    assert call(reps=1) == 1                  # k = 2 distinct choices need two replicas
    assert call(reps=513) == 1
    assert call(offsets=None) == 1 and call(thresholds=None) == 1
    assert call(hidden=96, dtype=1) == 1      # e4m3 rows need H % 128 == 0
    assert call(dtype=1, scales=None) == 1    # e4m3 needs the scales
    assert call(dtype=7) == 3                 # unsupported output type
    assert call(hidden=48) == 1               # H % 32
    assert call(expand_x=FAKE + 8) == 1       # misaligned output rows


def test_plain_c_program_uses_the_abi(tmp_path):
    """The header compiles as C99 and a C program links the library and gets
    the documented results from every host-side call (no GPU needed)."""
    import combine_moe_dispatch_layout_amd as m
    lib = m.library_path()
    exe = tmp_path / "abi_host_check"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_host_check.c"), "-o", str(exe),
                    lib, f"-Wl,-rpath,{os.path.dirname(lib)}"], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.strip() == "ok"


def test_dispatch_fused_rules(lib):
    def call(x=FAKE, xs=64, bs=4, h=64, ids=FAKE, k=2, e=8, align=128, counts=FAKE, send=FAKE,
             idx=FAKE, ex=FAKE, es=64, cap=64, dtype=0, qs=None, ws=None, wsb=0):
        return lib.moe_dispatch_fused(x, xs, bs, h, ids, k, e, align, counts, send, idx, ex, es,
                                      cap, dtype, qs, None, ws, wsb, None)

    assert call(dtype=5) == 3              # unknown dtype
    assert call(k=9) == 1                  # k > num_experts
    assert call(align=3) == 1              # align not a power of two
    assert call(h=48, xs=48, es=48) == 1   # hidden % 32
    assert call(dtype=1) == 1              # e4m3 needs hidden % 128 and scales
    assert call(h=128, xs=128, es=128, dtype=1) == 1   # e4m3 without scales
    assert call(counts=None) == 1
    assert call(x=FAKE + 2) == 1           # misaligned rows
    assert call(cap=-1) == 1
    # beyond one workgroup's pairs the two-launch path needs the workspace
    assert call(bs=4096, k=8, e=256) == 2


def test_dispatch_fused_noalloc_rules(lib):
    """The no-allocation entry point refuses, before any HIP call, a batch
    whose layout workspace exceeds its static scratch, and otherwise applies
    moe_dispatch_fused's argument rules."""
    lib.moe_noalloc_scratch_bytes.restype = ctypes.c_size_t
    scratch = lib.moe_noalloc_scratch_bytes()
    assert scratch == 5 << 20
    assert lib.moe_dispatch_layout_workspace_size((1 << 20) // 8, 8, 512) <= scratch

    def call(bs=4, k=2, e=8, dtype=0, cap=64, counts=FAKE):
        return lib.moe_dispatch_fused_noalloc(FAKE, 64, bs, 64, FAKE, k, e, 128, counts, FAKE,
                                              FAKE, FAKE, 64, cap, dtype, None, None, None)

    assert lib.moe_dispatch_layout_workspace_size(170000, 8, 512) > scratch
    assert call(bs=170000, k=8, e=512) == 5   # beyond the scratch
    assert lib.moe_status_string(5).decode().startswith("batch needs more")
    assert call(dtype=5) == 3                  # then the fused call's own rules
    assert call(k=9) == 1
    assert call(counts=None) == 1
    assert call(cap=-1) == 1


def test_probe_rules(lib):
    def call(items=4, row_bytes=64, reads=1, writes=8, src_total=4, dst_total=32, src=FAKE,
             dst=FAKE, src_rows=None, dst_rows=None):
        return lib.moe_probe_stream_mix(src, src_total, dst, dst_total, items, row_bytes, reads,
                                        writes, src_rows, dst_rows, None)

    assert call(reads=0) == 1 and call(writes=17) == 1
    assert call(row_bytes=24) == 1                 # not a multiple of 16
    assert call(dst_total=31) == 1                 # contiguous writes overrun dst
    assert call(src_total=3) == 1                  # contiguous reads overrun src
    assert call(src=FAKE + 8) == 1                 # misaligned
    assert call(items=0, src=None, dst=None) == 0  # nothing to do


def test_time_next_launches_rules(lib):
    """Binding rules of the kernel-timing hook.  Only host state is touched:
    the bound handles are never launched with (dropped again with n = 0)."""
    arr = ctypes.c_void_p * 17
    starts = arr(*[FAKE + 16 * i for i in range(17)])
    stops = arr(*[FAKE + 4096 + 16 * i for i in range(17)])
    assert lib.moe_time_unused_launches() == 0
    assert lib.moe_time_next_launches(starts, stops, -1) == 1
    assert lib.moe_time_next_launches(starts, stops, 17) == 1     # at most 16 pairs
    assert lib.moe_time_next_launches(None, stops, 2) == 1
    with_null = arr(FAKE, None)
    assert lib.moe_time_next_launches(starts, with_null, 2) == 1  # NULL among the first n
    assert lib.moe_time_unused_launches() == 0                    # failures bind nothing
    assert lib.moe_time_next_launches(starts, stops, 3) == 0
    assert lib.moe_time_unused_launches() == 3
    assert lib.moe_time_next_launches(None, None, 0) == 0         # drop
    assert lib.moe_time_unused_launches() == 0


def test_binding_fails_loudly_without_the_library(tmp_path):
    """No CPU fallback: with the library absent, loading it raises (in a
    fresh interpreter whose library path points at an empty folder)."""
    code = (
        "import combine_moe_dispatch_layout_amd as m, os\n"
        f"m._LIB_PATH = os.path.join({str(tmp_path)!r}, 'libmoe_dispatch.so')\n"
        "m._lib = None\n"
        "try:\n"
        "    m.load_library()\n"
        "except ImportError as e:\n"
        "    print('raised:', e)\n"
        "else:\n"
        "    print('loaded')\n")
    out = subprocess.run(["python", "-c", code], capture_output=True, text=True, cwd=ROOT,
                         timeout=120)
    assert "raised:" in out.stdout and "no CPU fallback" in out.stdout, out.stdout + out.stderr
