"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/cce.h declares, sizes its workspace consistently, and rejects bad
arguments synchronously, before any launch (so no device is touched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cce.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
FAKE = 0x100000          # aligned, never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def L():
    import linear_cross_entropy_forward_amd as M
    return M.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cce_\w+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"cce_forward", "cce_backward", "cce_workspace_size", "cce_read_stats"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared in cce.h but not exported"


def test_status_strings_and_tiles(L):
    for s in (OK, INVALID, UNSUPPORTED, WORKSPACE, -4, 99):
        assert L.cce_status_string(s)
    import linear_cross_entropy_forward_amd as M
    bn, bv, pw = M.tile_shape()
    assert bn == 256 and bv == 256 and pw == 128 and bv % pw == 0
    for k in range(17):
        assert L.cce_kernel_name(k) != b"unknown"
    assert L.cce_kernel_name(17) == b"unknown"


def test_state_and_workspace_size(L):
    st, ws = L.cce_state_size, L.cce_workspace_size
    assert st(-1, 64, 100, 0) == 0 and st(4, 64, 100, 7) == 0 and st(4, 0, 100, 0) == 0
    assert ws(-1, 64, 100, 0, 0) == 0 and ws(4, 64, 100, 7, 0) == 0 and ws(4, 64, 100, 0, 100) == 0
    assert st(0, 64, 100, 0) > 0 and ws(0, 64, 100, 0, 0) > 0  # an empty batch: the counters
    # the forward state: N x ceil(V/128) (max, sum-exp) partials dominate; at
    # the 8B head it stays under 45 MB (the loss-path overhead O(N + N V / 128))
    part = 4096 * ((128256 + 127) // 128) * 8
    s8 = st(4096, 4096, 128256, 0)
    assert part < s8 < 45e6
    # the backward workspace: 4 vocabulary chunks of G (<= 256 MiB) plus e^T and
    # the fp32 dE accumulation; the whole vocabulary in one chunk is larger
    a = ws(4096, 4096, 128256, 0, 0)
    whole = ws(4096, 4096, 128256, 0, 128256 + 256 - 128256 % 256)
    assert 256 << 20 < a < 450e6 < whole
    assert ws(4096, 4096, 128256, 0, 1024) < a
    assert ws(4096, 4096, 128256, 1, 0) >= ws(4096, 4096, 128256, 0, 0) // 2


def test_vocab_chunk(L):
    vc = L.cce_vocab_chunk
    assert vc(-1, 64, 100, 0, 0) == 0 and vc(4, 64, 100, 7, 0) == 0 and vc(4, 64, 100, 0, 100) == 0
    assert vc(4, 0, 100, 0, 0) == 0
    d = vc(4096, 4096, 128256, 0, 0)
    assert d % 256 == 0 and 256 <= d <= 128256 + 255
    # the default keeps a chunk's gradient tiles G within 256 MiB (bf16 stores
    # them once, fp32 in both orientations) but at least 8192 columns wide,
    # in nearly equal chunks of whole tiles: 4 chunks of 126 tiles at N = 4096
    assert d == 126 * 256 and 4096 * d * 2 <= 256 << 20
    assert vc(16384, 4096, 128256, 0, 0) == 8192
    assert vc(65536, 4096, 128256, 0, 0) == 8192 and 65536 * 8192 * 2 < 1 << 31
    assert vc(4096, 4096, 128256, 1, 0) == 8192 and 2 * 4096 * 8192 * 4 <= 256 << 20
    # ... and a chunk's classifier rows below 2^31 bytes: a classifier larger
    # than that (Gemma-2-27B's 256000 x 4608 bf16, 2.4 GB) is taken in chunks
    big = vc(1024, 4608, 256000, 0, 0)
    assert big % 256 == 0 and big * 4608 * 2 < 1 << 31 and big < 256000
    assert vc(4096, 4096, 128256, 0, 1024) == 1024
    assert vc(64, 64, 1000, 1, 0) == 1024          # clamped to the vocabulary, in whole tiles
    assert vc(64, 64, 1000, 1, 4096) == 1024


def _fwd(L, e=FAKE, c=FAKE, t=FAKE, N=64, D=64, V=100, dt=0, ign=-100, red=2, cap=0.0, loss=FAKE, lse=FAKE,
         ws=FAKE, wsb=1 << 30, bias=None, ls=0.0, zl=0.0):
    # ws / wsb: the forward state
    return L.cce_forward(e, c, bias, t, N, D, V, dt, ign, red, cap, ls, zl, loss, lse, None, ws, wsb, None)


def _bwd(L, e=FAKE, N=64, D=64, V=100, dt=0, red=2, cap=0.0, flt=1, acc=0, chunk=0, dE=FAKE, wsb=1 << 30,
         bias=None, db=None, ls=0.0, zl=0.0, gdt=0, stb=1 << 30, ws=FAKE, state=FAKE):
    return L.cce_backward(e, FAKE, bias, FAKE, N, D, V, dt, -100, red, cap, ls, zl, FAKE, FAKE, flt, acc, chunk, gdt,
                          dE, FAKE, db, state, stb, ws, wsb, None)


def test_forward_argument_errors(L):
    assert _fwd(L, e=None) == INVALID
    assert _fwd(L, t=None) == INVALID
    assert _fwd(L, loss=None) == INVALID
    assert _fwd(L, lse=None) == INVALID
    assert _fwd(L, ws=None) == INVALID
    assert _fwd(L, N=-1) == INVALID and _fwd(L, D=-1) == INVALID and _fwd(L, V=0) == INVALID
    # an empty batch is valid (null e / targets allowed); its size checks still apply
    assert _fwd(L, N=0, e=None, t=None, lse=None, wsb=16) == WORKSPACE
    assert L.cce_state_size(0, 64, 100, 0) > 0 and L.cce_state_size(-1, 64, 100, 0) == 0
    assert _fwd(L, dt=2) == INVALID
    assert _fwd(L, red=3) == INVALID
    assert _fwd(L, e=FAKE + 4) == INVALID            # misaligned
    for cap in (-1.0, float("inf"), float("nan")):  # softcap negative or not finite
        assert _fwd(L, cap=cap) == INVALID
    assert _fwd(L, cap=30.0, ls=0.1) == UNSUPPORTED    # soft-capping with label smoothing
    assert _fwd(L, cap=30.0, zl=1e-4, wsb=16) == WORKSPACE  # a valid cap passes to the size check
    assert _fwd(L, cap=30.0, dt=1) == UNSUPPORTED      # soft-capping is built for bf16 only
    assert _fwd(L, D=60) == UNSUPPORTED             # bf16 rows must be 16-byte multiples
    assert _fwd(L, dt=1, D=62) == UNSUPPORTED
    assert _fwd(L, wsb=16) == WORKSPACE
    assert _fwd(L, bias=FAKE + 1) == INVALID         # bias not aligned to its element
    assert _fwd(L, dt=1, bias=FAKE + 2) == INVALID
    for ls in (-0.1, 1.5, float("nan")):            # label smoothing outside [0, 1]
        assert _fwd(L, ls=ls) == INVALID
    for zl in (-1e-4, float("inf"), float("nan")):  # z-loss weight negative or not finite
        assert _fwd(L, zl=zl) == INVALID
    assert _fwd(L, ls=1.0, zl=1e-4, wsb=16) == WORKSPACE   # valid terms pass to the size check


def test_backward_argument_errors(L):
    assert _bwd(L, e=None) == INVALID
    assert _bwd(L, dE=FAKE + 8) == INVALID          # outputs 16-byte aligned
    assert _bwd(L, bias=FAKE + 1) == INVALID
    assert _bwd(L, db=FAKE + 2) == INVALID          # dbias is float
    assert _bwd(L, ls=2.0) == INVALID and _bwd(L, zl=-1.0) == INVALID
    assert _bwd(L, flt=2) == INVALID
    assert _bwd(L, acc=5) == INVALID
    assert _bwd(L, chunk=100) == INVALID
    # dE, dC, dbias each optional, but one of them is needed
    assert L.cce_backward(FAKE, FAKE, None, FAKE, 64, 64, 100, 0, -100, 2, 0.0, 0.0, 0.0, FAKE, FAKE, 1, 0, 0, 0,
                          None, None, None, FAKE, 1 << 30, FAKE, 1 << 30, None) == INVALID
    assert L.cce_backward(FAKE, FAKE, None, FAKE, 64, 64, 100, 0, -100, 2, 0.0, 0.0, 0.0, FAKE, FAKE, 1, 0, 0, 0,
                          None, FAKE, None, FAKE, 1 << 30, FAKE, 1024, None) == WORKSPACE
    # the state and the workspace are both required, each checked against its size
    assert _bwd(L, state=None) == INVALID and _bwd(L, ws=None) == INVALID
    assert _bwd(L, ws=FAKE + 8) == INVALID
    assert _bwd(L, stb=L.cce_state_size(64, 64, 100, 0) - 1) == WORKSPACE
    assert _bwd(L, gdt=2) == INVALID and _bwd(L, gdt=-1) == INVALID   # grad dtype: float32 or operand
    assert _bwd(L, gdt=1, wsb=1024) == WORKSPACE
    assert _bwd(L, cap=-1.0) == INVALID
    assert _bwd(L, cap=1.0, ls=0.2) == UNSUPPORTED
    assert _bwd(L, cap=1.0, wsb=1024) == WORKSPACE
    assert _bwd(L, wsb=1024) == WORKSPACE
    need = L.cce_workspace_size(64, 64, 100, 0, 0)
    assert _bwd(L, wsb=need - 1) == WORKSPACE


def test_size_limits(L):
    # operands addressed from one base must stay below 2 GiB
    assert _fwd(L, N=1 << 20, D=1024) == UNSUPPORTED
    assert _fwd(L, N=(1 << 20) + 256, D=8) == UNSUPPORTED


def test_stats_and_profile_argument_errors(L):
    import linear_cross_entropy_forward_amd as M
    st = M._Stats()
    assert L.cce_read_stats(None, 1024, 1, 1, None, ctypes.byref(st)) == INVALID
    assert L.cce_read_stats(FAKE, 8, 1, 1, None, ctypes.byref(st)) == INVALID
    assert L.cce_profile_start(-1, 4) == INVALID
    assert L.cce_profile_start(17, 4) == INVALID
    assert L.cce_profile_start(0, 0) == INVALID
    ms, n = ctypes.c_double(), ctypes.c_int()
    assert L.cce_profile_stop(17, ctypes.byref(ms), ctypes.byref(n)) == INVALID


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    import linear_cross_entropy_forward_amd as M
    e = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(M.CCEError):
        M.forward(e, e, torch.zeros(4, dtype=torch.int64))


def test_c_caller_builds(tmp_path):
    """The plain-C caller (tests/c_abi) compiles and links against the
    library through include/cce.h alone (it runs in the GPU tests)."""
    from linear_cross_entropy_forward_amd import build as b
    out = b.build_c_check(str(tmp_path / "cce_abi_check"))
    assert os.path.exists(out)


def test_bench_refuses_several_gpus():
    """The benchmark runs on one GPU: asked for more it prints why and exits
    non-zero, before touching a device."""
    import json
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_noalloc_forward_refuses_before_any_launch(L):
    """The no-allocation forward checks its sizes before any HIP call: a state
    beyond the static array (64 MiB) and invalid sizes are refused on a
    machine without a GPU."""
    N, D, V = 8192, 64, 256000
    assert L.cce_state_size(N, D, V, 0) > 64 << 20
    assert L.cce_forward_noalloc(FAKE, FAKE, None, FAKE, N, D, V, 0, -100, 2, 0.0, 0.0, 0.0, FAKE, FAKE, None,
                                 None) == WORKSPACE
    assert L.cce_forward_noalloc(FAKE, FAKE, None, FAKE, 64, 0, 100, 0, -100, 2, 0.0, 0.0, 0.0, FAKE, FAKE, None,
                                 None) == INVALID
