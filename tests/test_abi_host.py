"""Host-side checks of the C ABI (no GPU compute).

libcoda.so must load and export every function include/coda.h declares, and argument
errors must be reported before anything is enqueued. Every call here fails
validation (or is an M == 0 no-op), so no kernel is launched and no device memory is
touched; the fake pointers are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import transformer_gemm_epilogue_amd as coda
from transformer_gemm_epilogue_amd.build import LIB_PATH

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "coda.h")

OK, NULL, SHAPE, ALIGN, WS, HIP, ARG = 0, 1, 2, 3, 4, 5, 6
P = 0x100000  # a 16-byte aligned fake device address (never dereferenced)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(coda_\w+)\s*\(", text, flags=re.M)))


SPREAD = 1 << 36  # every fake buffer gets a region of its own this large


class Spread:
    """The library, called with each fake pointer argument (P + a small offset) moved to
    a region of its own: argument i at P + i * 2^36, offset kept. No two fake buffers
    then overlap, so the overlap rule stays out of the way of the check under test."""

    def __init__(self, lib):
        self._lib = lib

    def __getattr__(self, name):
        fn = getattr(self._lib, name)

        def call(*args):
            return fn(*[P + i * SPREAD + (a - P) if isinstance(a, int) and P <= a < P + 64 else a
                        for i, a in enumerate(args)])
        return call


@pytest.fixture(scope="module")
def raw():
    if not os.path.exists(LIB_PATH):
        pytest.fail("libcoda.so is not built: run __graft_entry__.build() first")
    return coda.lib()


@pytest.fixture(scope="module")
def L(raw):
    return Spread(raw)


def test_header_declares_the_entry_points():
    names = header_functions()
    for need in ("coda_gemm_rmsnorm_fwd", "coda_rowstat_reduce", "coda_gemm_rope", "coda_gemm_swiglu",
                 "coda_gemm_rmsnorm_bwd_stats"):
        assert need in names


def test_library_exports_every_declared_symbol(raw):
    missing = [n for n in header_functions() if not hasattr(raw, n)]
    assert not missing, missing


def test_binding_covers_every_declared_symbol():
    declared = set(header_functions()) - {"coda_status_string", "coda_build_source_hash"}
    assert declared == set(coda.SIGNATURES)


def test_binding_exports_every_public_wrapper():
    # every public wrapper of an entry point is listed for `from ... import *`
    import inspect
    public = {n for n, f in inspect.getmembers(coda, inspect.isfunction)
              if f.__module__ == coda.__name__ and not n.startswith("_")}
    assert public <= set(coda.__all__), sorted(public - set(coda.__all__))


def test_status_strings(L):
    for st in range(7):
        assert L.coda_status_string(st)
    assert L.coda_abi_version() == 103


def test_num_partials(L):
    for width, nb in ((1, 1), (256, 1), (257, 2), (4096, 16), (6144, 24)):
        assert coda.num_partials(width) == nb
    out = ctypes.c_int(0)
    assert L.coda_rowstat_num_partials(0, ctypes.byref(out)) == SHAPE
    assert L.coda_rowstat_num_partials(8, None) == NULL


def fwd(L, x=P, w0=P, z=P, g=P, w1=P, M=256, K=256, D=256, N1=256, eps=1e-6, h1=P, h2=P, part=P, r=P, y=P):
    return L.coda_gemm_rmsnorm_fwd(x, w0, z, g, w1, M, K, D, N1, eps, h1, h2, part, r, y, None)


def test_fwd_validation(L):
    assert fwd(L, x=None) == NULL
    assert fwd(L, y=None) == NULL
    assert fwd(L, K=100) == SHAPE          # not a multiple of 8
    assert fwd(L, D=0) == SHAPE
    assert fwd(L, N1=(1 << 22) + 8) == SHAPE
    assert fwd(L, M=-1) == SHAPE
    assert fwd(L, x=P + 8) == ALIGN
    assert fwd(L, h2=P + 2) == ALIGN
    assert fwd(L, eps=-1.0) == ARG
    assert fwd(L, eps=float("nan")) == ARG
    assert fwd(L, eps=float("inf")) == ARG
    assert fwd(L, M=0) == OK               # empty batch: nothing to do


def test_rope_validation(L):
    def call(M=64, K=64, n_q=128, n_k=128, n_v=128, hd=128, seq=64, off=0, cos=P, sin=P):
        return L.coda_gemm_rope(P, P, cos, sin, M, K, n_q, n_k, n_v, hd, seq, off, P, None)
    assert call(cos=None) == NULL
    assert call(hd=12) == SHAPE
    assert call(n_q=64) == SHAPE           # not a multiple of head_dim
    assert call(n_q=0, n_k=0, n_v=0) == SHAPE
    assert call(seq=0) == ARG
    assert call(off=-1) == ARG
    assert call(cos=P + 4) == ALIGN
    assert call(M=0) == OK
    # each rotary table must stay below 2^31 bytes: seq_len * head_dim <= 2^29
    assert call(hd=128, seq=(1 << 22) + 8, n_q=128, n_k=0, n_v=0) == SHAPE
    assert call(hd=128, seq=(1 << 22), n_q=128, n_k=0, n_v=0, M=0) == OK
    for name in ("coda_gemm_rope_persistent", "coda_gemm_rope_bwd"):
        fn = getattr(L, name)
        assert fn(P, P, P, P, 64, 64, 128, 0, 0, 128, (1 << 22) + 8, 0, P, None) == SHAPE
        assert fn(P, P, None, P, 64, 64, 128, 128, 128, 128, 64, 0, P, None) == NULL


def test_row_count_bound(L):
    """M above 2^24 rows is rejected by every GEMM entry point before anything is
    enqueued (with widths <= 2^22 this keeps tile counts below 2^30)."""
    big = (1 << 24) + 1
    assert L.coda_baseline_gemm(P, P, big, 64, 256, 1, P, None) == SHAPE
    assert L.coda_gemm_swiglu(P, P, big, 64, 128, P, None) == SHAPE
    assert L.coda_gemm_rope(P, P, P, P, big, 64, 128, 128, 128, 128, 64, 0, P, None) == SHAPE
    assert L.coda_gemm_rmsnorm_bwd_stats(P, P, P, big, 256, 256, P, P, P, None) == SHAPE
    assert L.coda_rowstat_reduce(P, big, 16, 4096, 1e-5, 0, P, None) == SHAPE
    assert L.coda_gemm_cross_entropy(P, P, P, big, 64, 256, P, P, P, P, None) == SHAPE
    nb = ctypes.c_int(0)
    assert L.coda_colstat_num_partials(big, ctypes.byref(nb)) == SHAPE


def test_swiglu_validation(L):
    assert L.coda_gemm_swiglu(P, P, 64, 64, 12, P, None) == SHAPE
    assert L.coda_gemm_swiglu(P, P, 64, 64, 0, P, None) == SHAPE
    assert L.coda_gemm_swiglu(P, None, 64, 64, 16, P, None) == NULL
    assert L.coda_gemm_swiglu(P, P, 64, 60, 16, P, None) == SHAPE
    assert L.coda_gemm_swiglu(P, P, 0, 64, 16, P, None) == OK


def test_bwd_validation(L):
    assert L.coda_gemm_rmsnorm_bwd_stats(P, P, P, 64, 64, 64, P, P, None, None) == NULL
    assert L.coda_gemm_rmsnorm_bwd_stats(P, P, P, 64, 63, 64, P, P, P, None) == SHAPE
    assert L.coda_gemm_rmsnorm_bwd_stats(P, P, P + 8, 64, 64, 64, P, P, P, None) == ALIGN
    assert L.coda_gemm_rmsnorm_bwd_stats(P, P, P, 0, 64, 64, P, P, P, None) == OK


def test_rowstat_validation(L):
    assert L.coda_rowstat_reduce(P, 64, 0, 64, 0.0, 0, P, None) == SHAPE
    assert L.coda_rowstat_reduce(P, 64, 4, 0, 0.0, 0, P, None) == SHAPE
    assert L.coda_rowstat_reduce(P, 64, 4, 64, 0.0, 7, P, None) == ARG
    assert L.coda_rowstat_reduce(P, 64, 4, 64, -1.0, 0, P, None) == ARG
    assert L.coda_rowstat_reduce(P + 2, 64, 4, 64, 0.0, 0, P, None) == ALIGN
    assert L.coda_rowstat_reduce(P, 0, 4, 64, 0.0, 0, P, None) == OK


def test_rope_tables_validation(L):
    assert L.coda_rope_tables(P, P, 0, 128, 1e4, None) == SHAPE
    assert L.coda_rope_tables(P, P, 16, 7, 1e4, None) == SHAPE
    assert L.coda_rope_tables(P, P, 16, 128, 0.0, None) == ARG
    assert L.coda_rope_tables(None, P, 16, 128, 1e4, None) == NULL


def test_baseline_validation(L):
    assert L.coda_baseline_gemm(P, P, 64, 60, 64, 1, P, None) == SHAPE
    assert L.coda_baseline_copy(P, P, 15, None) == SHAPE
    assert L.coda_baseline_copy(P, None, 16, None) == NULL
    assert L.coda_baseline_residual_rmsnorm(P, P, P, 64, 12, 1e-5, P, P, P, None) == SHAPE


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((8, 8), dtype=torch.bfloat16)
    with pytest.raises((ValueError, RuntimeError)):
        coda.coda_gemm_swiglu(x, torch.zeros((8, 16), dtype=torch.bfloat16))


def test_rmsnorm_bwd_validation(L):
    t = ctypes.c_int(-1)
    assert L.coda_colstat_num_partials(513, ctypes.byref(t)) == OK and t.value == 3
    assert L.coda_colstat_num_partials(0, ctypes.byref(t)) == OK and t.value == 0
    assert L.coda_colstat_num_partials(-1, ctypes.byref(t)) == SHAPE
    assert L.coda_colstat_num_partials(8, None) == NULL
    # output-side statistic
    assert L.coda_rowdot_stat(P, P, 64, 12, 64, P, None) == SHAPE        # N % 8 != 0
    assert L.coda_rowdot_stat(P, P, 64, 64, 0, P, None) == SHAPE         # d < 1
    assert L.coda_rowdot_stat(P, P, -1, 64, 64, P, None) == SHAPE
    assert L.coda_rowdot_stat(None, P, 64, 64, 64, P, None) == NULL
    assert L.coda_rowdot_stat(P + 8, P, 64, 64, 64, P, None) == ALIGN
    assert L.coda_rowdot_stat(P, P, 64, 64, 64, P + 2, None) == ALIGN
    assert L.coda_rowdot_stat(None, None, 0, 64, 64, None, None) == OK   # empty batch: no-op
    # column reduction
    assert L.coda_colsum_reduce(P, -1, 64, P, None) == SHAPE
    assert L.coda_colsum_reduce(P, 2, 0, P, None) == SHAPE
    assert L.coda_colsum_reduce(None, 2, 64, P, None) == NULL
    assert L.coda_colsum_reduce(P, 2, 64, None, None) == NULL
    assert L.coda_colsum_reduce(P + 2, 2, 64, P, None) == ALIGN
    # grad GEMM with the RMSNorm-backward epilogue
    #        dy w1 h1 gamma r  s  g_res   M   D   N  dh1 pgamma
    good = [P, P, P, P, P, P, None, 64, 64, 64, P, P, None]
    def dx(**kw):
        a = list(good)
        names = ["dy", "w1", "h1", "gamma", "r", "s", "g_res", "M", "D", "N", "dh1", "pgamma", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return L.coda_gemm_rmsnorm_bwd_dx(*a)
    assert dx(D=12) == SHAPE and dx(N=4) == SHAPE and dx(M=-1) == SHAPE
    for k in ("dy", "w1", "h1", "gamma", "r", "s", "dh1", "pgamma"):
        assert dx(**{k: None}) == NULL, k
    assert dx(h1=P + 8) == ALIGN and dx(g_res=P + 8) == ALIGN and dx(r=P + 2) == ALIGN
    assert dx(M=0, dy=None, w1=None, h1=None, gamma=None, r=None, s=None, dh1=None, pgamma=None) == OK
    # the combined call validates before launching anything
    full = [P, P, P, P, P, P, None, 64, 64, 64, P, P, P, P, None]
    bad = list(full); bad[5] = None      # y
    assert L.coda_rmsnorm_bwd(*bad) == NULL
    bad = list(full); bad[13] = None     # dgamma
    assert L.coda_rmsnorm_bwd(*bad) == NULL
    bad = list(full); bad[13] = P + 2
    assert L.coda_rmsnorm_bwd(*bad) == ALIGN
    bad = list(full); bad[8] = 20        # D % 8
    assert L.coda_rmsnorm_bwd(*bad) == SHAPE


def test_cross_entropy_validation(L):
    #        x  w  labels M   K   V  tile target lse loss stream
    good = [P, P, P, 64, 64, 64, P, P, P, P, None]
    names = ["x", "w", "labels", "M", "K", "V", "tile_lse", "target", "lse", "loss", "stream"]
    def ce(**kw):
        a = list(good)
        for k, v in kw.items():
            a[names.index(k)] = v
        return L.coda_gemm_cross_entropy(*a)
    assert ce(V=12) == SHAPE and ce(K=4) == SHAPE and ce(M=-1) == SHAPE
    for k in ("x", "w", "labels", "tile_lse", "target", "lse", "loss"):
        assert ce(**{k: None}) == NULL, k
    assert ce(x=P + 8) == ALIGN and ce(labels=P + 2) == ALIGN and ce(loss=P + 1) == ALIGN
    assert ce(M=0, x=None, w=None, labels=None, tile_lse=None, target=None, lse=None, loss=None) == OK
    # the merge alone: nb must match the vocabulary's tile count
    assert L.coda_lse_reduce(P, P, 64, 3, 512, P, P, P, None) == SHAPE
    assert L.coda_lse_reduce(None, P, 64, 2, 512, P, P, P, None) == NULL
    assert L.coda_lse_reduce(P, P, 0, 2, 512, None, None, None, None) == OK


def test_overlapping_buffers_are_rejected(raw):
    """Outputs may overlap neither an input nor another output (CODA_ERR_ARG, before
    anything is enqueued). The ranges are the buffers' true byte sizes: sharing a buffer's
    last 16 bytes is refused. (Adjacent buffers and inputs that alias each other pass;
    that needs a launch, so the GPU tests cover it.)"""
    M, K, D, N1 = 256, 512, 256, 264
    b = 1 << 40
    def at(i):
        return b + i * SPREAD
    x, w0, z, g, w1, h1, h2, part, r, y = (at(i) for i in range(10))
    def fwd(**kw):
        a = dict(x=x, w0=w0, z=z, g=g, w1=w1, h1=h1, h2=h2, part=part, r=r, y=y)
        a.update(kw)
        return raw.coda_gemm_rmsnorm_fwd(a["x"], a["w0"], a["z"], a["g"], a["w1"], M, K, D, N1, 1e-5, a["h1"],
                                         a["h2"], a["part"], a["r"], a["y"], None)
    h1_bytes = M * D * 2
    assert fwd(h2=h1) == ARG                      # two outputs on one buffer
    assert fwd(h2=h1 + h1_bytes - 16) == ARG      # last 16 bytes of h1 shared
    assert fwd(y=x + 16) == ARG                   # output inside an input
    assert fwd(r=w1) == ARG
    assert fwd(part=z) == ARG
    assert fwd(h1=g + D * 2 - 16) == ARG          # h1 starts in the last 16 bytes of gamma
    assert raw.coda_gemm_residual_rmsnorm_partials(x, w0, z, g, M, K, D, h1, x, part, None) == ARG
    assert raw.coda_gemm_rowscale(h2, w1, r, M, D, N1, h2, None) == ARG
    # the stages' GEMM2 input h2 and r are outputs of the earlier stages: overlapping them is refused
    assert fwd(h2=y) == ARG
    assert raw.coda_gemm_swiglu(x, w0, M, K, 64, x + 2 * M * K - 16, None) == ARG   # last 16 bytes of x
    assert raw.coda_gemm_swiglu(x, x, M, K, 64, x, None) == ARG
    assert raw.coda_rowstat_reduce(part, M, 16, 4096, 1e-5, 0, part + 4 * (16 * M - 1), None) == ARG
    assert raw.coda_gemm_rmsnorm_bwd_stats(x, w0, z, M, D, K, z, part, r, None) == ARG    # dh2 on h2
    assert raw.coda_gemm_rmsnorm_bwd_stats(x, w0, z, M, D, K, h1, part, part, None) == ARG  # s on partials
    assert raw.coda_gemm_rope(x, w0, z, g, M, K, 128, 128, 0, 128, 64, 0, g, None) == ARG  # out on a table
    assert raw.coda_gemm_cross_entropy(x, w0, z, M, K, 512, part, r, r, y, None) == ARG     # target == lse
    assert raw.coda_gemm_cross_entropy(x, w0, z, M, K, 512, part, z, r, y, None) == ARG     # target on labels
    assert raw.coda_lse_reduce(part, z, M, 2, 512, r, y, part, None) == ARG                 # loss on tile_lse
    assert raw.coda_rowdot_stat(x, w0, M, K, K, x, None) == ARG
    assert raw.coda_colsum_reduce(part, 4, 256, part + 4 * 256 * 3, None) == ARG
    assert raw.coda_baseline_copy(x, x + 16, 64, None) == ARG
    assert raw.coda_baseline_gemm(x, w0, M, K, N1, 1, w0, None) == ARG
    assert raw.coda_gemm_swiglu_bwd(x, w0, z, M, K, 64, z, None) == ARG
    assert raw.coda_rope_tables(g, g + 4 * 8, 16, 128, 1e4, None) == ARG


def test_noalloc_capacity_and_arguments(L):
    def call(M=256, K=256, D=256, N1=256, eps=1e-5, x=P, h1=P, r=P):
        return L.coda_gemm_rmsnorm_fwd_noalloc(x, P, P, P, P, M, K, D, N1, eps, h1, P, r, P, None)
    cap = coda.NOALLOC_SCRATCH_FLOATS
    assert call(M=cap // 16 + 1, D=4096) == WS     # 16 partials per row past the array
    assert call(M=cap + 1, D=256) == WS
    assert call(M=-1) == SHAPE and call(K=12) == SHAPE and call(N1=0) == SHAPE
    assert call(eps=-1.0) == ARG
    assert call(M=0, x=None, h1=None, r=None) == OK


def test_library_matches_its_sources(raw, tmp_path):
    """The loaded library was built from the sources next to it; a copy of those sources
    with one edited file no longer matches, and the check refuses it."""
    import shutil
    coda.check_source_hash(raw)            # the in-tree build is current
    shutil.copytree(os.path.join(ROOT, "transformer_gemm_epilogue_amd", "csrc"),
                    tmp_path / "transformer_gemm_epilogue_amd" / "csrc")
    shutil.copytree(os.path.join(ROOT, "include"), tmp_path / "include")
    coda.check_source_hash(raw, str(tmp_path))   # an unedited copy matches
    src = tmp_path / "transformer_gemm_epilogue_amd" / "csrc" / "coda_aux.hip"
    src.write_text(src.read_text() + "\n// edited\n")
    with pytest.raises(coda.StaleLibraryError):
        coda.check_source_hash(raw, str(tmp_path))


def test_schedule_probe_validation(L, raw):
    f = ctypes.c_float(0.125)
    assert L.coda_baseline_schedule_probe(-1, 5, 1, f, 0, P, P + 16, None) == SHAPE
    assert L.coda_baseline_schedule_probe(8, 5, 1, f, 0, P, P + 16, None) == SHAPE
    assert L.coda_baseline_schedule_probe(7, 5, 1, f, 0, P, P + 16, None) == ARG      # fill != 0
    assert L.coda_baseline_schedule_probe(7, 5, 1, ctypes.c_float(0.0), 3, P, P + 16, None) == ARG  # seed != 0
    assert L.coda_baseline_schedule_probe(0, 0, 1, f, 0, P, P + 16, None) == SHAPE
    assert L.coda_baseline_schedule_probe(0, 5, 0, f, 0, P, P + 16, None) == SHAPE
    assert L.coda_baseline_schedule_probe(0, 5, 65536, f, 0, P, P + 16, None) == SHAPE
    assert L.coda_baseline_schedule_probe(0, 5, 1, f, 0, None, P + 16, None) == NULL
    assert L.coda_baseline_schedule_probe(0, 5, 1, f, 0, P, None, None) == NULL
    assert L.coda_baseline_schedule_probe(0, 5, 1, f, 0, P + 2, P + 16, None) == ALIGN
    assert L.coda_baseline_schedule_probe(0, 5, 1, f, 0, P, P + 20, None) == ALIGN
    # out [512] fp32 and cycles [8] int64 overlapping
    assert raw.coda_baseline_schedule_probe(0, 5, 1, f, 0, P, P + 64, None) == ARG


def test_split_forward_validation(L):
    out = ctypes.c_int64(-1)
    assert L.coda_gemm_rmsnorm_fwd_workspace_bytes(8, 8, 8, 8, None) == NULL
    assert L.coda_gemm_rmsnorm_fwd_workspace_bytes(-1, 8, 8, 8, ctypes.byref(out)) == SHAPE
    assert L.coda_gemm_rmsnorm_fwd_workspace_bytes(8, 12, 8, 8, ctypes.byref(out)) == SHAPE
    assert L.coda_gemm_rmsnorm_fwd_workspace_bytes(0, 8, 8, 8, ctypes.byref(out)) == OK and out.value == 0
    f = ctypes.c_float(1e-5)
    args = [P, P, P, P, P, 8, 8, 8, 8]
    outs = [P, P, P, P, P]
    assert L.coda_gemm_rmsnorm_fwd_ws(*args, ctypes.c_float(-1.0), *outs, P, 0, None) == ARG
    assert L.coda_gemm_rmsnorm_fwd_ws(*args, f, *outs, P, -1, None) == ARG
    assert L.coda_gemm_rmsnorm_fwd_ws(None, P, P, P, P, 8, 8, 8, 8, f, *outs, P, 0, None) == NULL
    assert L.coda_gemm_rmsnorm_fwd_ws(P, P, P, P, P, 8, 12, 8, 8, f, *outs, P, 0, None) == SHAPE
    assert L.coda_gemm_rmsnorm_fwd_ws(P, P, P, P, P, 0, 8, 8, 8, f, *outs, None, 0, None) == OK


def test_split_rope_swiglu_validation(L):
    out = ctypes.c_int64(-1)
    assert L.coda_split_workspace_bytes(8, 8, 8, None) == NULL
    assert L.coda_split_workspace_bytes(8, 12, 8, ctypes.byref(out)) == SHAPE
    assert L.coda_split_workspace_bytes(0, 8, 8, ctypes.byref(out)) == OK and out.value == 0
    assert L.coda_gemm_swiglu_ws(P, P, 8, 8, 8, P, P, -1, None) == ARG
    assert L.coda_gemm_swiglu_ws(None, P, 8, 8, 8, P, P, 0, None) == NULL
    assert L.coda_gemm_swiglu_ws(P, P, 8, 8, 12, P, P, 0, None) == SHAPE
    assert L.coda_gemm_swiglu_ws(P, P, 0, 8, 8, P, None, 0, None) == OK
    rope = [P, P, P, P, 8, 8, 8, 8, 8, 8, 8, 0, P]
    assert L.coda_gemm_rope_ws(*rope, P, -1, None) == ARG
    assert L.coda_gemm_rope_ws(None, *rope[1:], P, 0, None) == NULL
    assert L.coda_gemm_rope_ws(P, P, P, P, 0, 8, 8, 8, 8, 8, 8, 0, P, None, 0, None) == OK


def test_split_backward_and_cross_entropy_validation(L):
    # a negative workspace size is refused before any pointer is read (all NULL here)
    N0 = None
    assert L.coda_gemm_rmsnorm_bwd_stats_ws(N0, N0, N0, 8, 8, 8, N0, N0, N0, N0, -1, None) == ARG
    assert L.coda_gemm_rmsnorm_bwd_stats_ws(N0, P, P, 8, 8, 8, P, P, P, P, 0, None) == NULL
    assert L.coda_gemm_rmsnorm_bwd_stats_ws(P, P, P, 8, 12, 8, P, P, P, P, 0, None) == SHAPE
    assert L.coda_gemm_rmsnorm_bwd_stats_ws(N0, N0, N0, 0, 8, 8, N0, N0, N0, N0, 0, None) == OK
    dx = [P, P, P, P, P, P, None]
    assert L.coda_gemm_rmsnorm_bwd_dx_ws(*([N0] * 7), 8, 8, 8, N0, N0, N0, -1, None) == ARG
    assert L.coda_gemm_rmsnorm_bwd_dx_ws(N0, *dx[1:], 8, 8, 8, P, P, P, 0, None) == NULL
    assert L.coda_gemm_rmsnorm_bwd_dx_ws(*dx, 8, 12, 8, P, P, P, 0, None) == SHAPE
    assert L.coda_gemm_rmsnorm_bwd_dx_ws(*([N0] * 7), 0, 8, 8, N0, N0, N0, 0, None) == OK
    assert L.coda_gemm_swiglu_bwd_ws(N0, N0, N0, 8, 8, 8, N0, N0, -1, None) == ARG
    assert L.coda_gemm_swiglu_bwd_ws(N0, P, P, 8, 8, 8, P, P, 0, None) == NULL
    assert L.coda_gemm_swiglu_bwd_ws(P, P, P, 8, 8, 12, P, P, 0, None) == SHAPE
    assert L.coda_gemm_swiglu_bwd_ws(N0, N0, N0, 0, 8, 8, N0, N0, 0, None) == OK
    assert L.coda_gemm_cross_entropy_ws(N0, N0, N0, 8, 8, 8, N0, N0, N0, N0, N0, -1, None) == ARG
    assert L.coda_gemm_cross_entropy_ws(N0, P, P, 8, 8, 8, P, P, P, P, P, 0, None) == NULL
    assert L.coda_gemm_cross_entropy_ws(P, P, P, 8, 8, 12, P, P, P, P, P, 0, None) == SHAPE
    assert L.coda_gemm_cross_entropy_ws(N0, N0, N0, 0, 8, 8, N0, N0, N0, N0, N0, 0, None) == OK
    rope = [P, P, P, P, 8, 8, 8, 8, 8, 8, 8, 0, P]
    assert L.coda_gemm_rope_bwd_ws(*rope, P, -1, None) == ARG
    assert L.coda_gemm_rope_bwd_ws(None, *rope[1:], P, 0, None) == NULL
    assert L.coda_gemm_rope_bwd_ws(P, P, P, P, 0, 8, 8, 8, 8, 8, 8, 0, P, None, 0, None) == OK


def test_split_plan_rules(L):
    """The split-depth plan, on the host for a given CU count (no device needed)."""
    plan = coda.coda_split_plan
    tile = 256 * 1024                      # bytes of one fp32 partial tile
    # at most half as many tiles as CUs: every tile split, S <= CUs / T, <= 8, >= 16 steps
    assert plan(1024, 4096, 14336, 256) == (4, 112, 0, 64 * 4 * tile)      # 64 tiles, 448 steps
    assert plan(1024, 6144, 4096, 256) == (2, 64, 0, 96 * 2 * tile)        # 96 tiles: 2, not 3
    assert plan(300, 264, 4128, 256) == (8, 18, 0, 4 * 8 * tile)           # 129 steps: 8 x 18, last 3
    assert plan(300, 264, 992, 256) == (1, 31, 0, 0)                       # 31 steps: no 2 x 16
    assert plan(300, 264, 1000, 256) == (2, 16, 0, 4 * 2 * tile)           # 32 steps, the last ragged
    assert plan(40, 8, 8, 256) == (1, 1, 0, 0)                             # one step
    # more than half: a partial last wave of r <= CUs / 2 tiles is split, slices >= 32 steps
    assert plan(4096, 6144, 4096, 256) == (2, 64, 256, 128 * 2 * tile)     # 384 tiles: 256 + 128
    assert plan(4096, 4608, 8192, 256) == (8, 32, 256, 32 * 8 * tile)      # 288 tiles: 256 + 32
    assert plan(4096, 5120, 2048, 256) == (2, 32, 256, 64 * 2 * tile)
    assert plan(4096, 5120, 1024, 256) == (1, 32, 0, 0)                    # 32 steps: no 2 x 32
    assert plan(8192, 4096, 14336, 256) == (1, 448, 0, 0)                  # 512 tiles: full waves
    assert plan(4096, 12288, 4096, 256) == (1, 128, 0, 0)                  # 768 tiles
    assert plan(1024, 12288, 4096, 256) == (1, 128, 0, 0)                  # 192 tiles: 3/4 of the CUs
    # the plan follows the CU count
    assert plan(1024, 4096, 14336, 304) == (4, 112, 0, 64 * 4 * tile)
    assert plan(1024, 4096, 14336, 128) == (2, 224, 0, 64 * 2 * tile)
    assert plan(0, 4096, 14336, 256)[3] == 0
    out = ctypes.c_int(0)
    i64 = ctypes.c_int64(0)
    assert L.coda_split_plan(8, 8, 8, 0, ctypes.byref(out), ctypes.byref(out), ctypes.byref(out),
                             ctypes.byref(i64)) == ARG
    assert L.coda_split_plan(8, 12, 8, 256, ctypes.byref(out), ctypes.byref(out), ctypes.byref(out),
                             ctypes.byref(i64)) == SHAPE
    assert L.coda_split_plan(8, 8, 8, 256, None, ctypes.byref(out), ctypes.byref(out), ctypes.byref(i64)) == NULL
