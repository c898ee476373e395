"""Host-side checks of libspec_verify.so that need no GPU.

The library loads, exports every entry point include/spec_verify.h declares, and its
host argument checks reject bad calls before anything is enqueued.  No call here
reaches a kernel launch.
"""
import ctypes
import os
import re

import pytest

import exact_rejection_sampling_amd as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")

OK, EINVAL, EDTYPE, EWORKSPACE = 0, 1, 2, 3
NULL = ctypes.c_void_p(0)
FAKE = ctypes.c_void_p(0x1000)       # never dereferenced: every call below fails on the host


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = sv.load_library()
    names = declared_functions()
    assert {"spec_verify_chain", "spec_verify_greedy", "spec_verify_tree"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared but not exported"


def test_abi_version_and_strings():
    lib = sv.load_library()
    assert lib.spec_abi_version() == 2
    for c in range(6):
        assert lib.spec_status_string(c)
    for c in range(8):
        assert lib.spec_req_status_string(c)


def test_workspace_sizes():
    lib = sv.load_library()
    n = lib.spec_chain_workspace_bytes(64, 5, 128256)
    # one 8-byte summary per wave (at most one per 2048-element chunk, the wave count
    # rounded up to whole 4-wave blocks) per row, plus per-request decisions, gathered
    # draft values (3 words per draft) and 4096-element chunk masses: well under a megabyte
    rows, P, S2 = 64 * 6, (128256 + 2047) // 2048, (128256 + 4095) // 4096
    assert rows * 4 * 8 <= n < rows * (P + 3) * 8 + 64 * (16 + 3 * 5 * 8 + S2 * 8) + 4096
    assert lib.spec_chain_workspace_bytes(0, 5, 128256) == 256   # the counter header only
    assert lib.spec_chain_workspace_bytes(1, 64, 10) == 0      # gamma above the limit
    assert lib.spec_chain_workspace_bytes(1, 5, 0) == 0
    assert lib.spec_greedy_workspace_bytes(256, 8, 128256) > 0
    assert lib.spec_tree_workspace_bytes(32, 63, 152064) > 0
    assert lib.spec_tree_workspace_bytes(32, 5000, 152064) == 0  # N above the limit


def _chain(lib, *, B=2, gamma=2, V=16, T=1.0, ldt=0, qdt=0, logits=FAKE, q=FAKE, tok=FAKE, u=FAKE,
           acc=FAKE, out=FAKE, st=FAKE, ws=NULL, wsn=0):
    return lib.spec_verify_chain(logits, ldt, q, qdt, tok, u, B, gamma, V, ctypes.c_float(T),
                                 acc, out, st, NULL, ws, wsn, NULL)


def test_chain_host_validation():
    lib = sv.load_library()
    assert _chain(lib, B=-1) == EINVAL
    assert _chain(lib, gamma=-1) == EINVAL
    assert _chain(lib, gamma=64) == EINVAL
    assert _chain(lib, V=0) == EINVAL
    for T in (0.0, -1.0, float("nan"), float("inf"), 1e-9, 1e9):
        assert _chain(lib, T=T) == EINVAL
    assert _chain(lib, ldt=7) == EDTYPE
    assert _chain(lib, qdt=-1) == EDTYPE
    assert _chain(lib, B=0, logits=NULL, q=NULL, tok=NULL, u=NULL, acc=NULL, out=NULL, st=NULL) == OK
    assert _chain(lib, logits=NULL) == EINVAL
    assert _chain(lib, u=NULL) == EINVAL
    assert _chain(lib, q=NULL) == EINVAL
    assert _chain(lib, gamma=0, q=NULL, tok=NULL) == EWORKSPACE    # gamma 0 needs no drafts
    assert _chain(lib, ws=NULL, wsn=1 << 20) == EWORKSPACE
    assert _chain(lib, ws=ctypes.c_void_p(0x1001), wsn=1 << 20) == EWORKSPACE   # misaligned
    assert _chain(lib, ws=ctypes.c_void_p(0x10000), wsn=8) == EWORKSPACE        # too small


def test_greedy_and_tree_host_validation():
    lib = sv.load_library()
    g = lambda **k: lib.spec_verify_greedy(k.get("l", FAKE), k.get("dt", 1), k.get("t", FAKE),
                                            k.get("B", 2), k.get("G", 2), k.get("V", 16),
                                            FAKE, FAKE, FAKE, k.get("ws", NULL), k.get("wsn", 0), NULL)
    assert g(B=-1) == EINVAL and g(G=64) == EINVAL and g(V=0) == EINVAL
    assert g(dt=3) == EDTYPE and g(l=NULL) == EINVAL and g(t=NULL) == EINVAL
    assert g(G=0, t=NULL) == EWORKSPACE and g(B=0, l=NULL) == OK
    t = lambda **k: lib.spec_verify_tree(k.get("l", FAKE), k.get("dt", 1), FAKE, k.get("par", FAKE),
                                          FAKE, k.get("B", 2), k.get("N", 5), k.get("V", 16),
                                          ctypes.c_float(k.get("T", 1.0)), FAKE, FAKE, FAKE, FAKE,
                                          NULL, 0, NULL)
    assert t(N=0) == EINVAL and t(N=4097) == EINVAL and t(T=0.0) == EINVAL
    assert t(dt=2) == EDTYPE and t(par=NULL) == EINVAL and t(B=0, l=NULL) == OK
    assert t() == EWORKSPACE


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(2, 3, 8)
    with pytest.raises(ValueError, match="GPU"):
        sv.spec_verify_greedy(x, torch.zeros(2, 2, dtype=torch.int32))


def test_product_path_does_not_import_the_oracle():
    """The package and its library never touch oracle/ (no CPU fallback)."""
    pkg = os.path.join(ROOT, "exact_rejection_sampling_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            path = os.path.join(dirpath, f)
            if f.endswith(".py"):
                src = open(path).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", src, flags=re.M), path
            elif f.endswith((".hip", ".h", ".cpp")):
                assert "oracle" not in open(path).read().lower(), path


def test_grid_limit():
    # a dispatch counts work-items in 32 bits: at most 16777215 blocks of 256 threads
    lib = sv.load_library()
    big_rows = (1 << 22, 7, 16)        # 2^25 rows, one block each at least
    assert lib.spec_chain_workspace_bytes(*big_rows) == 0
    assert lib.spec_greedy_workspace_bytes(*big_rows) == 0
    assert _chain(lib, B=1 << 22, gamma=7, V=16) == EINVAL
    assert lib.spec_chain_workspace_bytes(1 << 20, 7, 16) > 0      # 2^23 rows fit
    assert lib.spec_tree_workspace_bytes(1 << 22, 4, 1 << 20) == 0  # 2^22 * 128 blocks
    assert lib.spec_tree_workspace_bytes(1 << 16, 4, 1 << 20) > 0


def test_tree_residual_host_validation():
    lib = sv.load_library()
    r = lambda **k: lib.spec_verify_tree_residual(
        k.get("l", FAKE), k.get("dt", 1), k.get("q", FAKE), k.get("qdt", 0), FAKE, k.get("par", FAKE),
        k.get("ua", FAKE), k.get("ud", FAKE), k.get("B", 2), k.get("N", 5), k.get("V", 16),
        ctypes.c_float(k.get("T", 1.0)), FAKE, FAKE, FAKE, FAKE, k.get("ws", NULL), k.get("wsn", 0), NULL)
    assert r(N=0) == EINVAL and r(N=4097) == EINVAL and r(T=float("nan")) == EINVAL
    assert r(V=(1 << 21) + 1) == EINVAL and r(V=1 << 21) == EWORKSPACE   # chunk masses staged on chip
    assert r(dt=2) == EDTYPE and r(qdt=5) == EDTYPE
    assert r(q=NULL) == EINVAL and r(ud=NULL) == EINVAL and r(ua=NULL) == EINVAL
    assert r(B=0, l=NULL) == OK and r() == EWORKSPACE
    assert lib.spec_tree_residual_workspace_bytes(2, 5, (1 << 21) + 1) == 0
    n = lib.spec_tree_residual_workspace_bytes(32, 31, 32000)
    assert n > lib.spec_tree_workspace_bytes(32, 31, 32000)   # plus the pass descriptors


def test_stop_variants_host_validation():
    lib = sv.load_library()
    c = lambda **k: lib.spec_verify_chain_stop(
        FAKE, 0, FAKE, 0, FAKE, FAKE, k.get("B", 2), 2, 16, ctypes.c_float(1.0),
        k.get("stop", FAKE), k.get("n", 1), k.get("budget", NULL), FAKE, FAKE, FAKE, k.get("fin", NULL), NULL,
        NULL, 0, NULL)
    assert c(n=-1) == EINVAL and c(n=257) == EINVAL and c(stop=NULL) == EINVAL
    assert c(n=0, stop=NULL) == EWORKSPACE and c(n=256) == EWORKSPACE   # only the workspace is missing
    assert c(budget=FAKE, fin=FAKE) == EWORKSPACE and c(B=0) == OK
    g = lambda **k: lib.spec_verify_greedy_stop(
        FAKE, 1, FAKE, k.get("B", 2), 2, 16, k.get("stop", FAKE), k.get("n", 1), NULL, FAKE, FAKE, FAKE,
        NULL, NULL, 0, NULL)
    assert g(n=-1) == EINVAL and g(n=257) == EINVAL and g(stop=NULL) == EINVAL
    assert g(n=0, stop=NULL) == EWORKSPACE and g(B=0) == OK


def test_tree_greedy_host_validation():
    lib = sv.load_library()
    t = lambda **k: lib.spec_verify_tree_greedy(k.get("l", FAKE), k.get("dt", 1), FAKE, k.get("par", FAKE),
                                                 k.get("B", 2), k.get("N", 5), k.get("V", 16),
                                                 FAKE, FAKE, FAKE, FAKE, NULL, 0, NULL)
    assert t(N=0) == EINVAL and t(N=4097) == EINVAL and t(V=0) == EINVAL
    assert t(dt=2) == EDTYPE and t(par=NULL) == EINVAL and t(l=NULL) == EINVAL
    assert t(B=0, l=NULL) == OK and t() == EWORKSPACE


def test_options_entry_points_host_validation():
    lib = sv.load_library()
    from exact_rejection_sampling_amd._binding import SpecOptions
    bad = SpecOptions()
    bad.n_stop = 300
    c = lambda opt, **k: lib.spec_verify_chain_ex(FAKE, 0, FAKE, 0, FAKE, FAKE, k.get("B", 2), 2, 16,
                                                  ctypes.c_float(1.0), opt, FAKE, FAKE, FAKE, NULL, NULL, 0, NULL)
    assert c(None) == EWORKSPACE and c(ctypes.byref(SpecOptions())) == EWORKSPACE
    assert c(ctypes.byref(bad)) == EINVAL and c(None, B=0) == OK
    g = lambda opt: lib.spec_verify_greedy_ex(FAKE, 1, FAKE, 2, 2, 16, opt, FAKE, FAKE, FAKE, NULL, 0, NULL)
    assert g(None) == EWORKSPACE and g(ctypes.byref(bad)) == EINVAL
    sparse = SpecOptions()
    sparse.q_index, sparse.q_k = FAKE, 0
    assert c(ctypes.byref(sparse)) == EINVAL
    lazy = SpecOptions()
    lazy.lazy_rows = -1
    assert c(ctypes.byref(lazy)) == EINVAL
    for k in (1, 3, 100):
        lazy.lazy_rows = k
        assert c(ctypes.byref(lazy)) == EWORKSPACE


def test_trace_setter_refuses_outside_trace_builds():
    """spec_trace_set is exported by every build; only the trace build accepts a buffer."""
    lib = sv.load_library()
    assert lib.spec_trace_set(FAKE, 16) == EINVAL
    assert lib.spec_trace_set(NULL, 0) == EINVAL


def test_static_scratch_entry_rejects_sizes_past_its_scratch():
    """spec_verify_chain_static checks sizes before it touches a device: sizes whose
    workspace exceeds SPEC_STATIC_SCRATCH_BYTES get SPEC_ESCRATCH, invalid ones EINVAL."""
    lib = sv.load_library()
    ESCRATCH = 5
    big = lib.spec_chain_workspace_bytes(8192, 5, 128256)
    assert big > (4 << 20)
    args = (FAKE, 1, FAKE, 0, FAKE, FAKE)
    tail = (ctypes.c_float(1.0), FAKE, FAKE, FAKE, NULL, NULL)
    assert lib.spec_verify_chain_static(*args, 8192, 5, 128256, *tail) == ESCRATCH
    assert lib.spec_verify_chain_static(*args, 4, 64, 128, *tail) == EINVAL     # gamma above the limit
    assert lib.spec_status_string(ESCRATCH)
