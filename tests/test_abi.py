"""The C ABI library on the CPU: it loads, exports every function that
include/*.h declares, and rejects invalid arguments on the host, before any
HIP call (so none of these tests needs a GPU or launches a kernel)."""

import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

from draft_token_verification_chain_amd import _binding as bnd  # noqa: E402

OK, INVALID, WS_SMALL, UNSUPPORTED, HIPERR = range(5)
F32, BF16 = 0, 1
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails before any use


@pytest.fixture(scope="module")
def lib():
    # These calls pass placeholder pointers that validation must reject; with a
    # GPU present a validation slip would launch on them, so run only where no
    # device is visible.
    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("host-validation tests run where no GPU is visible")
    from draft_token_verification_chain_amd import build as b

    if b.is_stale():
        b.build(verbose=False)
    return bnd.load()


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(sv_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for must in ("sv_verify_chain", "sv_verify_greedy", "sv_verify_tree", "sv_chain_workspace_bytes",
                 "sv_greedy_workspace_bytes", "sv_tree_workspace_bytes", "sv_status_string", "sv_version"):
        assert must in names


def test_library_exports_every_declared_function(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.sv_version() >= 100
    for s in range(5):
        assert bnd.status_string(s).startswith("SV_")
    assert "unknown" in bnd.status_string(99)


def test_handoff_polls_setter(lib):
    # host state only: returns the previous bound; a negative value restores 65536
    first = lib.sv_set_handoff_polls(0)
    try:
        assert lib.sv_set_handoff_polls(17) == 0
        assert lib.sv_set_handoff_polls(-1) == 17
        assert lib.sv_set_handoff_polls(-5) == 65536
        assert bnd.set_handoff_polls(3) == 65536
        assert bnd.set_handoff_polls(-1) == 3
    finally:
        lib.sv_set_handoff_polls(first)


def test_workspace_queries(lib):
    a = lib.sv_chain_workspace_bytes(64, 4, 128256, BF16)
    b = lib.sv_chain_workspace_bytes(64, 4, 128256, F32)
    assert a > 0 and b >= a and a % 256 == 0
    assert lib.sv_chain_workspace_bytes(-1, 4, 10, F32) == 0
    assert lib.sv_chain_workspace_bytes(1, 65, 10, F32) == 0
    assert lib.sv_chain_workspace_bytes(1, 4, 0, F32) == 0
    assert lib.sv_chain_workspace_bytes(1, 4, 10, 7) == 0
    assert lib.sv_greedy_workspace_bytes(256, 5, 128256, BF16) > 0
    assert lib.sv_tree_workspace_bytes(16, 64, 128256, BF16) > 0
    assert lib.sv_tree_workspace_bytes(16, 1025, 128256, BF16) == 0
    # grows with every size
    assert lib.sv_chain_workspace_bytes(128, 4, 128256, BF16) > a
    assert lib.sv_chain_workspace_bytes(64, 8, 128256, BF16) > a


def _chain(lib, B=2, k=2, V=100, dt=F32, ws_bytes=None, **ptrs):
    p = dict(tokens=FAKE, draft=FAKE, target=FAKE, temp=FAKE, u=FAKE, acc=FAKE, em=FAKE, ap=None, ws=FAKE)
    p.update(ptrs)
    if ws_bytes is None:
        ws_bytes = max(lib.sv_chain_workspace_bytes(max(B, 0), max(k, 0), max(V, 1), dt if dt in (0, 1) else 0), 1)
    return lib.sv_verify_chain(B, k, V, dt, p["tokens"], p["draft"], p["target"], p["temp"], p["u"], p["acc"],
                               p["em"], p["ap"], p["ws"], ws_bytes, None)


def test_chain_rejects_bad_arguments_on_the_host(lib):
    assert _chain(lib, B=-1) == INVALID
    assert _chain(lib, k=-1) == INVALID
    assert _chain(lib, V=0) == INVALID
    assert _chain(lib, dt=5) == INVALID
    assert _chain(lib, k=65) == UNSUPPORTED
    assert _chain(lib, V=(1 << 30) + 1) == UNSUPPORTED
    for key in ("target", "temp", "u", "acc", "em", "tokens", "draft"):
        assert _chain(lib, **{key: None}) == INVALID, key
    assert _chain(lib, ws_bytes=16) == WS_SMALL
    assert _chain(lib, ws=None) == INVALID
    assert _chain(lib, ws=ctypes.c_void_p(0x1004)) == INVALID  # not 16-byte aligned


def test_chain_empty_batch_and_k0_pointer_rules(lib):
    # B == 0: nothing to do, no pointer is looked at
    assert _chain(lib, B=0, target=None, temp=None, u=None, acc=None, em=None, ws=None, ws_bytes=0) == OK
    # k == 0 still needs every other pointer (a k == 0 call that passes validation
    # would launch, so only failing calls are made here; the GPU tests run k == 0)
    assert _chain(lib, k=0, tokens=None, draft=None, em=None) == INVALID
    assert _chain(lib, k=0, tokens=None, draft=None, temp=None) == INVALID


def test_chain_static_rejects_bad_arguments_on_the_host(lib):
    """sv_verify_chain_static: the same argument checks as sv_verify_chain, and
    sizes whose workspace exceeds SV_STATIC_WORKSPACE_BYTES refused, all
    before the device lookup (no HIP call)."""
    def cs(B=2, k=3, V=50, dt=BF16, tokens=FAKE, draft=FAKE, target=FAKE, temp=FAKE, u=FAKE, acc=FAKE, em=FAKE):
        return lib.sv_verify_chain_static(B, k, V, dt, tokens, draft, target, temp, u, acc, em, None, None)

    assert cs(B=-1) == INVALID
    assert cs(k=-1) == INVALID
    assert cs(dt=5) == INVALID
    assert cs(k=65) == UNSUPPORTED
    for key in ("target", "temp", "u", "acc", "em", "tokens", "draft"):
        assert cs(**{key: None}) == INVALID, key
    assert cs(B=0, target=None, temp=None, u=None, acc=None, em=None) == OK
    # the largest batch that fits, and the first one that does not
    static = 16 << 20
    B = 1
    while lib.sv_chain_workspace_bytes(2 * B, 4, 128256, BF16) <= static:
        B *= 2
    lo, hi = B, 2 * B
    while hi - lo > 1:
        mid = (lo + hi) // 2
        lo, hi = (mid, hi) if lib.sv_chain_workspace_bytes(mid, 4, 128256, BF16) <= static else (lo, mid)
    assert lib.sv_chain_workspace_bytes(hi, 4, 128256, BF16) > static
    assert cs(B=hi, k=4, V=128256) == WS_SMALL


def test_greedy_rejects_bad_arguments_on_the_host(lib):
    def g(B=2, k=3, V=50, dt=BF16, tokens=FAKE, target=FAKE, acc=FAKE, em=FAKE, ws=FAKE, ws_bytes=1 << 20):
        return lib.sv_verify_greedy(B, k, V, dt, tokens, target, acc, em, ws, ws_bytes, None)

    assert g(B=-1) == INVALID
    assert g(k=-2) == INVALID
    assert g(V=-3) == INVALID
    assert g(dt=2) == INVALID
    assert g(k=100) == UNSUPPORTED
    assert g(tokens=None) == INVALID
    assert g(target=None) == INVALID
    assert g(ws_bytes=8) == WS_SMALL
    assert g(B=0, tokens=None, target=None, acc=None, em=None, ws=None, ws_bytes=0) == OK


def test_tree_rejects_bad_arguments_on_the_host(lib):
    def t(B=2, N=8, V=50, dt=F32, tok=FAKE, par=FAKE, stride=0, md=3, target=FAKE, acc=FAKE, em=FAKE,
          nodes=None, ws=FAKE, ws_bytes=1 << 20):
        return lib.sv_verify_tree(B, N, V, dt, tok, par, stride, md, target, acc, em, nodes, ws, ws_bytes, None)

    assert t(N=0) == INVALID
    assert t(md=-1) == INVALID
    assert t(stride=4) == INVALID  # a per-sequence parent stride shorter than N
    assert t(stride=-1) == INVALID
    assert t(N=1025) == UNSUPPORTED
    assert t(md=(1 << 24) + 1) == UNSUPPORTED
    assert t(par=None) == INVALID
    assert t(tok=None) == INVALID
    assert t(ws_bytes=8) == WS_SMALL
    assert t(B=0, tok=None, par=None, target=None, acc=None, em=None, ws=None, ws_bytes=0) == OK


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(bnd, "_lib", None)
    monkeypatch.setattr(bnd, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        bnd.load()


def test_commit_rejects_bad_arguments_on_the_host(lib):
    def c(B=4, width=3, acc=FAKE, em=FAKE, sl=FAKE, hist=FAKE, stride=8):
        return lib.sv_commit_tokens(B, width, acc, em, sl, hist, stride, None, None, None, None)

    assert c(B=-1) == INVALID
    assert c(width=0) == INVALID
    assert c(stride=-1) == INVALID
    assert c(B=(1 << 24) + 1) == UNSUPPORTED
    assert c(acc=None) == INVALID
    assert c(em=None) == INVALID
    assert c(sl=None) == INVALID
    assert c(B=0, acc=None, em=None, sl=None, hist=None) == OK


def test_tree_sampled_rejects_bad_arguments_on_the_host(lib):
    def t(B=2, N=8, V=50, dt=F32, tok=FAKE, par=FAKE, stride=0, md=3, draft=FAKE, target=FAKE, temp=FAKE, u=FAKE,
          acc=FAKE, em=FAKE, nodes=None, ws=FAKE, ws_bytes=1 << 20):
        return lib.sv_verify_tree_sampled(B, N, V, dt, tok, par, stride, md, draft, target, temp, u, acc, em, nodes,
                                          ws, ws_bytes, None)

    assert lib.sv_tree_sampled_workspace_bytes(16, 64, 128256, BF16) > 2 * lib.sv_tree_workspace_bytes(
        16, 64, 128256, BF16)
    assert lib.sv_tree_sampled_workspace_bytes(16, 1025, 128256, BF16) == 0
    assert t(B=-1) == INVALID
    assert t(N=0) == INVALID
    assert t(md=-1) == INVALID
    assert t(stride=4) == INVALID
    assert t(V=0) == INVALID
    assert t(dt=3) == INVALID
    assert t(N=1025) == UNSUPPORTED
    assert t(md=(1 << 30)) == UNSUPPORTED
    assert t(V=(1 << 20) + 1) == UNSUPPORTED
    for key in ("tok", "par", "draft", "target", "temp", "u", "acc", "em"):
        assert t(**{key: None}) == INVALID, key
    assert t(ws_bytes=8) == WS_SMALL
    assert t(ws=ctypes.c_void_p(0x1008)) == INVALID
    assert t(B=0, tok=None, par=None, draft=None, target=None, temp=None, u=None, acc=None, em=None, ws=None,
             ws_bytes=0) == OK


C_CONSUMER = r"""
#include <stdio.h>
#include <string.h>
#include "specverify.h"

int main(void) {
    if (sv_version() < 100) return 1;
    if (strncmp(sv_status_string(SV_ERR_INVALID_ARGUMENT), "SV_", 3) != 0) return 2;
    if (sv_chain_workspace_bytes(64, 4, 128256, SV_BF16) == 0) return 3;
    if (sv_tree_sampled_workspace_bytes(16, 64, 128256, SV_BF16) == 0) return 4;
    /* rejected on the host: no launch */
    if (sv_verify_chain(-1, 4, 100, SV_F32, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL)
        != SV_ERR_INVALID_ARGUMENT) return 5;
    if (sv_verify_greedy(2, SV_MAX_DRAFTS + 1, 100, SV_BF16, NULL, NULL, NULL, NULL, NULL, 0, NULL)
        != SV_ERR_UNSUPPORTED) return 6;
    /* an empty batch is a no-op */
    if (sv_verify_tree(0, 4, 100, SV_F32, NULL, NULL, 0, 3, NULL, NULL, NULL, NULL, NULL, 0, NULL) != SV_OK) return 7;
    if (sv_commit_tokens(0, 5, NULL, NULL, NULL, NULL, 0, NULL, NULL, NULL, NULL) != SV_OK) return 8;
    puts("ok");
    return 0;
}
"""


def test_header_is_plain_c_and_links(lib, tmp_path):
    """A C11 program includes include/specverify.h, links against the shared
    library and calls it (only calls that return before any launch)."""
    import shutil
    import subprocess

    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    src = tmp_path / "consumer.c"
    src.write_text(C_CONSUMER)
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(bnd.LIB_PATH)
    subprocess.check_call(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", str(src), "-o", str(exe),
                           "-L", libdir, "-lspecverify", f"-Wl,-rpath,{libdir}"])
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0 and out.stdout.strip() == "ok", (out.returncode, out.stdout, out.stderr)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits with a message (before
    any GPU work)."""
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
