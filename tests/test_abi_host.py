"""Host-side checks of the C ABI (CPU only: nothing here launches a kernel).

* libvmoba.so loads and exports every function include/vmoba.h declares;
* every argument error is reported before anything is enqueued;
* the fast division and the partition arithmetic of the kernels' geometry header
  agree with exact division and with the oracle's block table;
* the host code runs clean under the address and undefined-behaviour sanitizers.
"""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from block_sparse_attention_layer_amd import _lib
from block_sparse_attention_layer_amd._lib import CProblem, OPS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vmoba.h")
GEOM = os.path.join(ROOT, "block_sparse_attention_layer_amd", "csrc", "geometry.h")

NULL = ctypes.c_void_p(0)
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every case below fails on the host


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def _prob(**kw):
    base = dict(batch=1, heads=2, head_dim=64, T=4, H=8, W=8, layer_idx=2, bt=2, bh=4,
                bw=4, dtype=1, grad_dtype=1)
    base.update(kw)
    return CProblem(*[base[n] for n, _ in CProblem._fields_])


def test_header_symbols_exported(L):
    text = open(HEADER).read()
    names = set(re.findall(r"\b(vmoba_[a-z_]+)\s*\(", text))
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert L.vmoba_version().decode().startswith("vmoba")


@pytest.mark.parametrize("kw,code", [
    ({}, 0),
    ({"T": 5}, 2), ({"bt": 3}, 2), ({"H": 0}, 2), ({"batch": 0}, 2), ({"layer_idx": -1}, 2),
    ({"layer_idx": 0}, 3),                          # 1D block must hold whole frames
    ({"layer_idx": 1}, 3),                          # 2D block must span all frames
    ({"layer_idx": 0, "bt": 1, "bh": 8, "bw": 8}, 0),
    ({"layer_idx": 1, "bt": 4}, 0),
    ({"dtype": 7}, 5), ({"head_dim": 96}, 6), ({"grad_dtype": 0}, 5), ({"grad_dtype": 3}, 5),
    ({"dtype": 0, "grad_dtype": 0}, 0), ({"dtype": 0, "grad_dtype": 1}, 0),
    ({"T": 1024, "H": 1024, "W": 8, "bt": 1, "bh": 1, "bw": 8, "heads": 2}, 8),
])
def test_validate_codes(L, kw, code):
    p = _prob(**kw)
    assert L.vmoba_validate(ctypes.byref(p)) == code


def test_num_blocks_and_workspace(L):
    p = _prob()
    nb = ctypes.c_int32()
    assert L.vmoba_num_blocks(ctypes.byref(p), ctypes.byref(nb)) == 0
    assert nb.value == 8
    n = ctypes.c_size_t()
    for op in OPS.values():
        assert L.vmoba_workspace_size(ctypes.byref(p), op, ctypes.byref(n)) == 0
    assert L.vmoba_workspace_size(ctypes.byref(p), OPS["select"], ctypes.byref(n)) == 0
    assert n.value >= 2 * 64 * 4
    assert L.vmoba_workspace_size(ctypes.byref(p), 99, ctypes.byref(n)) == 10
    assert L.vmoba_num_blocks(ctypes.byref(p), None) == 1


def test_null_and_tau_and_workspace_errors(L):
    p = _prob()
    bp = ctypes.byref(p)
    assert L.vmoba_partition_pool(bp, NULL, FAKE, FAKE, FAKE, NULL) == 1
    assert L.vmoba_partition_pool(None, FAKE, FAKE, FAKE, FAKE, NULL) == 1
    # tau checked before pointers
    for tau in (0.0, -0.1, 1.5, float("nan"), float("inf")):
        assert L.vmoba_select(bp, NULL, NULL, tau, NULL, NULL, NULL, NULL, NULL, NULL,
                              NULL, 0, NULL) == 4
    assert L.vmoba_select(bp, FAKE, FAKE, 0.25, FAKE, FAKE, FAKE, NULL, FAKE, NULL, FAKE,
                          1 << 20, NULL) == 1
    # workspace too small / missing
    assert L.vmoba_select(bp, FAKE, FAKE, 0.25, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE,
                          16, NULL) == 7
    assert L.vmoba_select(bp, FAKE, FAKE, 0.25, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL,
                          1 << 20, NULL) == 1
    assert L.vmoba_sparse_attn_fwd(bp, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, NULL, 0,
                                   NULL) == 1
    assert L.vmoba_sparse_attn_bwd(bp, *([FAKE] * 13), NULL, 0, NULL) in (1, 7)
    assert L.vmoba_sparse_attn_bwd(bp, *([FAKE] * 14), 4, NULL) == 7
    assert L.vmoba_dense_attn_fwd(bp, FAKE, FAKE, NULL, FAKE, FAKE, NULL, 0, NULL) == 1
    assert L.vmoba_dense_attn_bwd(bp, *([FAKE] * 9), NULL, 0, NULL) == 7
    # bad problem wins over everything else
    bad = _prob(T=5)
    assert L.vmoba_sparse_attn_fwd(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, FAKE, 1 << 30, NULL) == 2


def test_noalloc_backward_host_errors(L):
    """The no-allocation backward rejects, before any HIP call: a bad problem, NULL
    pointers, too many blocks, and a problem whose delta rows exceed its fixed scratch."""
    bp = ctypes.byref(_prob())
    assert L.vmoba_sparse_attn_bwd_noalloc(ctypes.byref(_prob(T=5)), *([FAKE] * 13), NULL) == 2
    for i in range(13):
        args = [FAKE] * 13
        args[i] = NULL
        assert L.vmoba_sparse_attn_bwd_noalloc(bp, *args, NULL) == 1
    many = _prob(T=1, H=1, W=1025, bt=1, bh=1, bw=1, layer_idx=2)
    assert L.vmoba_sparse_attn_bwd_noalloc(ctypes.byref(many), *([FAKE] * 13), NULL) == 2
    # 8 x 12 heads x 75,600 tokens of fp32 delta = 29 MB > 16 MiB
    big = _prob(batch=8, heads=12, head_dim=128, T=21, H=45, W=80, bt=3, bh=9, bw=8,
                dtype=0, grad_dtype=0)
    assert L.vmoba_validate(ctypes.byref(big)) == 0
    assert 8 * 12 * 75600 * 4 > _lib.NOALLOC_SCRATCH_BYTES
    assert L.vmoba_sparse_attn_bwd_noalloc(ctypes.byref(big), *([FAKE] * 13), NULL) == 12
    assert b"scratch" in L.vmoba_status_string(12)


def test_too_many_blocks_rejected_by_sparse_calls(L):
    # 1025 blocks of one token: above the selection kernel's limit
    p = _prob(T=1, H=1, W=1025, bt=1, bh=1, bw=1, layer_idx=2)
    assert L.vmoba_validate(ctypes.byref(p)) == 0
    assert L.vmoba_select(ctypes.byref(p), FAKE, FAKE, 0.25, FAKE, FAKE, FAKE, FAKE, FAKE,
                          NULL, FAKE, 1 << 30, NULL) == 2
    assert L.vmoba_sparse_attn_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, FAKE, 1 << 30, NULL) == 2


_GEOM_PROG = r"""
#include <cstdio>
#include <cstdlib>
#include <cstdint>
#include <initializer_list>
#include "GEOM"
using namespace vmoba;
int main(int argc, char** argv) {
  if (argc > 1 && argv[1][0] == 'd') {
    // fast division against exact division
    unsigned long long bad = 0, n_checked = 0;
    uint64_t st = 88172645463325252ull;
    for (uint32_t d = 1; d < 4100; ++d) {
      FastDiv f = make_fastdiv(d);
      for (int i = 0; i < 3000; ++i) {
        st ^= st << 13; st ^= st >> 7; st ^= st << 17;
        uint32_t n = (i < 1000) ? uint32_t(i) : uint32_t(st & 0x7fffffffu);
        if (i == 1000) n = 0x7fffffffu;
        n_checked++;
        if (fd_div(n, f) != n / d) bad++;
      }
    }
    for (uint32_t d : {65535u, 65536u, 82944u, 122500u, 1000003u, 0x7fffffffu}) {
      FastDiv f = make_fastdiv(d);
      for (uint32_t n : {0u, 1u, d - 1, d, d + 1, 2 * d - 1, 0x7fffffffu}) {
        if (n > 0x7fffffffu) continue;
        n_checked++; if (fd_div(n, f) != n / d) bad++;
      }
    }
    printf("%llu %llu\n", n_checked, bad);
    return 0;
  }
  // token table: T H W bt bh bw
  int T = atoi(argv[1]), H = atoi(argv[2]), W = atoi(argv[3]);
  Geom g{};
  g.T = T; g.H = H; g.W = W; g.bt = atoi(argv[4]); g.bh = atoi(argv[5]); g.bw = atoi(argv[6]);
  g.nt = T / g.bt; g.nh = H / g.bh; g.nw = W / g.bw; g.Nb = g.nt * g.nh * g.nw;
  g.S = g.bt * g.bh * g.bw;
  g.div_S = make_fastdiv(g.S); g.div_nhnw = make_fastdiv(g.nh * g.nw);
  g.div_nw = make_fastdiv(g.nw); g.div_bhbw = make_fastdiv(g.bh * g.bw);
  g.div_bw = make_fastdiv(g.bw);
  for (int j = 0; j < g.Nb; ++j)
    for (int r = 0; r < g.S; ++r) printf("%d\n", block_base(g, j) + block_offset(g, r));
  return 0;
}
"""


@pytest.fixture(scope="module")
def geom_exe(tmp_path_factory):
    d = tmp_path_factory.mktemp("geom")
    src = d / "geom.cpp"
    src.write_text(_GEOM_PROG.replace("GEOM", GEOM))
    exe = d / "geom"
    subprocess.run(["g++", "-O2", "-std=c++17", str(src), "-o", str(exe)], check=True)
    return str(exe)


def test_fast_division_is_exact(geom_exe):
    out = subprocess.run([geom_exe, "d"], capture_output=True, text=True, check=True).stdout
    checked, bad = map(int, out.split())
    assert checked > 10_000_000 and bad == 0


@pytest.mark.parametrize("lat,block", [
    ((4, 8, 8), (2, 4, 4)), ((21, 30, 52), (1, 30, 52)), ((21, 30, 52), (21, 6, 4)),
    ((24, 36, 64), (4, 6, 8)), ((21, 45, 80), (3, 9, 8)), ((6, 18, 16), (3, 9, 8)),
])
def test_kernel_token_map_matches_oracle_blocks(geom_exe, lat, block):
    out = subprocess.run([geom_exe, *map(str, lat), *map(str, block)], capture_output=True,
                         text=True, check=True).stdout
    got = np.array(out.split(), dtype=np.int64)
    ref = oracle.block_members(*lat, block).reshape(-1)
    assert np.array_equal(got, ref)


SANITIZE_DIR = os.path.join(ROOT, "tests", "host_sanitize")
CSRC = os.path.join(ROOT, "block_sparse_attention_layer_amd", "csrc")


def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    """api.cpp and validate.cpp built by g++ with ASan and UBSan (aborting on the first
    report), linked against host stand-ins of the kernel launchers: every entry point with
    valid arguments and with each argument error, every op's workspace size, every status
    string, sizes near and far past the int32 limits, and the geometry helpers."""
    exe = tmp_path / "vmoba_host_sanitized"
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer"]
    cmd = ["g++", "-std=c++17", "-g", "-O1", *san, "-I", os.path.join(ROOT, "include"),
           os.path.join(SANITIZE_DIR, "driver.cpp"),
           os.path.join(SANITIZE_DIR, "stub_launchers.cpp"),
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "validate.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok")


def test_select_mode_errors(L):
    p = _prob()
    bp = ctypes.byref(p)
    args = lambda mode, tau, k, ws=FAKE, n=1 << 20: (bp, FAKE, FAKE, mode, tau, k, FAKE, FAKE,
                                                     FAKE, FAKE, FAKE, NULL, ws, n, NULL)
    assert L.vmoba_select_mode(*args(4, 0.25, 1)) == 11          # unknown mode
    assert L.vmoba_select_mode(*args(-1, 0.25, 1)) == 11
    for mode in (1, 3):                                           # top-k needs k >= 1
        assert L.vmoba_select_mode(*args(mode, 0.25, 0)) == 11
        assert L.vmoba_select_mode(*args(mode, 0.25, -5)) == 11
        assert L.vmoba_select_mode(*args(mode, float("nan"), 3, FAKE, 16)) == 7   # tau unused
    for mode in (0, 2):                                           # threshold needs a tau
        for tau in (0.0, 1.5, float("nan")):
            assert L.vmoba_select_mode(*args(mode, tau, 3)) == 4
        assert L.vmoba_select_mode(*args(mode, 0.25, 0, FAKE, 16)) == 7           # k unused
    assert L.vmoba_select_mode(*args(2, 0.25, 1, NULL, 1 << 20)) == 1
    assert L.vmoba_status_string(11).decode().startswith("unknown selection mode")
    # the local modes need the bitmap and row statistics behind the scores
    n = ctypes.c_size_t(0)
    assert L.vmoba_workspace_size(bp, 1, ctypes.byref(n)) == 0
    nb, groups = 8, p.batch * p.heads
    assert n.value >= groups * nb * nb * 4 + groups * nb * 4 + groups * nb * 12


def test_token_call_errors(L):
    """Token-granular calls: bf16 only, blocks of at least 4 tokens for the attention,
    tau in (0, 1], null pointers and workspace checked before anything is enqueued."""
    f32 = _prob()                                  # fp32 problem
    bf = _prob(dtype=0, grad_dtype=1)
    sel = lambda p, tau=0.25, ws=FAKE, n=1 << 30: L.vmoba_select_tokens(
        ctypes.byref(p), FAKE, FAKE, tau, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, n, NULL)
    assert sel(f32) == 5
    for tau in (0.0, 1.5, float("nan")):
        assert sel(bf, tau) == 4
    assert sel(bf, 0.25, FAKE, 16) == 7
    assert sel(bf, 0.25, NULL, 1 << 30) == 1
    fwd = lambda p, ws=FAKE, n=1 << 30: L.vmoba_token_attn_fwd(
        ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, n, NULL)
    bwd = lambda p, ws=FAKE, n=1 << 30: L.vmoba_token_attn_bwd(
        ctypes.byref(p), *([FAKE] * 14), ws, n, NULL)
    tiny_blocks = _prob(dtype=0, grad_dtype=1, bt=1, bh=1, bw=2)   # 2 tokens per block
    for call in (fwd, bwd):
        assert call(f32) == 5
        assert call(tiny_blocks) == 2
        assert call(bf, FAKE, 16) == 7
    # workspace: the list-position mask (and delta for the backward)
    n = ctypes.c_size_t(0)
    bp = ctypes.byref(bf)
    G, Lt, nb = 2, 256, 8
    assert L.vmoba_workspace_size(bp, OPS["token_fwd"], ctypes.byref(n)) == 0
    assert n.value >= G * Lt * 4
    assert L.vmoba_workspace_size(bp, OPS["token_bwd"], ctypes.byref(n)) == 0
    assert n.value >= G * Lt * 4 + G * Lt * 4
    assert L.vmoba_workspace_size(bp, OPS["select_tokens"], ctypes.byref(n)) == 0
    assert n.value >= G * Lt * nb * 4
