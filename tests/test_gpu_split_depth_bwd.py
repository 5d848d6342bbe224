"""The backward and cross-entropy GEMMs under the split-depth schedule (the *_ws entry
points), through the C ABI: each output has fewer 256 x 256 tiles than the GPU has CUs, so
each tile's depth is cut into slices whose fp32 partial tiles go to the caller's
workspace, and the same epilogue runs on their sum in slice order. Parity with the fp64
oracle on every element (ragged rows, features and depth; two and eight slices),
determinism from call to call, bit-identity with the one-kernel entry point when the
output is large enough that nothing splits, and graph replays equal to the eager call."""
import ctypes

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_util import assert_close, assert_close_tiles, bf16_bits, log, to_dev_bf16

pytestmark = pytest.mark.gpu
TIGHT = 1e-4  # fp32 outputs against fp64: relative Frobenius bound


@pytest.fixture(scope="module")
def coda():
    import torch
    import transformer_gemm_epilogue_amd as c
    assert torch.cuda.is_available()
    c.lib()
    return c


def sync():
    import torch
    torch.cuda.synchronize()


def dec(t):
    return O.decode_bf16(bf16_bits(t))


# ------------------------------------------------------------ RMSNorm backward statistic
@pytest.mark.parametrize("shape", [(300, 520, 1096), (517, 264, 4096)])
def test_bwd_stats_split_depth(coda, shape):
    M, D, N = shape
    assert coda.coda_split_workspace_bytes(M, D, N) > 0
    log(f"bwd_stats split M={M} D={D} N={N}")
    wl = W.bwd_stats(seed=90 + M % 7, M=M, D=D, N=N)
    dh2, part, s = coda.coda_gemm_rmsnorm_bwd_stats_ws(to_dev_bf16(wl["dy"]), to_dev_bf16(wl["w1"]),
                                                       to_dev_bf16(wl["h2"]))
    sync()
    ref = O.gemm_rmsnorm_bwd_stats(wl["dy"], wl["w1"], wl["h2"])
    assert_close_tiles("dh2", dec(dh2), ref["dh2"])
    assert_close_tiles("partials", part.cpu().numpy(), ref["partials"], rel_fro=TIGHT, tile_n=1)
    assert_close_tiles("s", s.cpu().numpy(), ref["s_prime"], rel_fro=TIGHT)


# ------------------------------------------------------------ RMSNorm backward, dh1 / dgamma
@pytest.mark.parametrize("shape", [(517, 392, 1064), (300, 264, 4096)])
def test_rmsnorm_bwd_dx_split_depth(coda, shape):
    """dh1 and the dgamma column partials from the grad GEMM dy W1^T split over its depth
    N, with s and r as the GPU path has them (the row-dot of dy and the forward's y)."""
    import torch
    M, D, N = shape
    assert coda.coda_split_workspace_bytes(M, D, N) > 0
    log(f"rmsnorm_bwd_dx split M={M} D={D} N={N}")
    wl = W.rmsnorm_bwd_full(93 + M % 5, M, D, N)
    dev = {k: to_dev_bf16(wl[k]) for k in ("h1", "gamma", "w1", "dy", "g_res")}
    h = dev["h1"].float()
    r = torch.rsqrt((h * h).mean(dim=1) + wl["eps"]).contiguous()
    h2 = (h * dev["gamma"].float()).to(torch.bfloat16).contiguous()
    y = coda.coda_gemm_rowscale(h2, dev["w1"], r)
    s = coda.coda_rowdot_stat(dev["dy"], y, D)
    dh1, part = coda.coda_gemm_rmsnorm_bwd_dx_ws(dev["dy"], dev["w1"], dev["h1"], dev["gamma"], r, s,
                                                 g_res=dev["g_res"])
    dgamma = coda.coda_colsum_reduce(part)
    sync()
    ref = O.rmsnorm_bwd(wl["h1"], wl["gamma"], wl["w1"], wl["dy"], wl["eps"], g_res=wl["g_res"])
    assert_close_tiles("dh1", dec(dh1), ref["dh1"])
    assert_close_tiles("dgamma_partials", part.cpu().numpy(), ref["dgamma_partials"], rel_fro=TIGHT, tile_m=1)
    assert_close("dgamma", dgamma.cpu().numpy(), ref["dgamma"], rel_fro=TIGHT)


# ------------------------------------------------------------ SwiGLU backward
@pytest.mark.parametrize("shape", [(333, 1040, 136), (300, 4096, 264),
                                   (300, 4128, 264)])   # 8 slices of 18 steps, the last of 3
def test_swiglu_bwd_split_depth(coda, shape):
    M, Dm, F = shape
    assert coda.coda_split_workspace_bytes(M, F, Dm) > 0
    log(f"swiglu_bwd split M={M} Dm={Dm} F={F}")
    wl = W.swiglu_bwd(seed=95 + M % 3, M=M, Dm=Dm, F=F)
    dh = coda.coda_gemm_swiglu_bwd_ws(to_dev_bf16(wl["dy"]), to_dev_bf16(wl["w_down"]), to_dev_bf16(wl["h"]))
    sync()
    ref = O.gemm_swiglu_bwd(wl["dy"], wl["w_down"], wl["h"])["dh"]
    got = dec(dh)
    assert_close_tiles("dG", got[:, 0::2], ref[:, 0::2])
    assert_close_tiles("dU", got[:, 1::2], ref[:, 1::2])


# ------------------------------------------------------------ RoPE backward
def test_rope_bwd_split_depth(coda):
    wl = W.rope_bwd(seed=97, M=300, K=1032, n_q=256, n_k=128, n_v=128, head_dim=128, seq_len=300, pos_offset=11)
    assert coda.coda_split_workspace_bytes(300, 512, 1032) > 0
    log("rope_bwd split M=300 K=1032 N=512")
    c, s = coda.coda_rope_tables(wl["seq_len"], wl["head_dim"], wl["theta"])
    out = coda.coda_gemm_rope_bwd_ws(to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"]), c, s, wl["n_q"], wl["n_k"],
                                     wl["n_v"], wl["head_dim"], wl["seq_len"], wl["pos_offset"])
    sync()
    ref = O.gemm_rope_bwd(wl["x"], wl["w"], wl["n_q"], wl["n_k"], wl["n_v"], wl["head_dim"], wl["seq_len"],
                          wl["pos_offset"], wl["theta"])
    assert_close_tiles("dqkv", dec(out), ref)


# ------------------------------------------------------------ cross-entropy
def run_ce(coda, wl, split=True):
    import torch
    labels = torch.from_numpy(wl["labels"]).cuda()
    fn = coda.coda_gemm_cross_entropy_ws if split else coda.coda_gemm_cross_entropy
    out = fn(to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"]), labels)
    sync()
    return [t.cpu().numpy() for t in out]


@pytest.mark.parametrize("shape", [(300, 1024, 1000), (40, 4096, 2056)])
def test_cross_entropy_split_depth(coda, shape):
    M, K, V = shape
    assert coda.coda_split_workspace_bytes(M, V, K) > 0
    log(f"cross_entropy split M={M} K={K} V={V}")
    wl = W.cross_entropy(seed=99 + M % 5, M=M, K=K, V=V, ignore_every=7)
    loss, lse, target, tile = run_ce(coda, wl)
    ref = O.gemm_cross_entropy(wl["x"], wl["w"], wl["labels"])
    assert_close_tiles("tile_lse", tile, ref["tile_lse"], rel_fro=TIGHT, tile_n=1)
    assert_close_tiles("lse", lse, ref["lse"], rel_fro=TIGHT)
    assert_close_tiles("target", target, ref["target"], rel_fro=TIGHT)
    assert_close_tiles("loss", loss, ref["loss"], rel_fro=TIGHT)
    assert np.all(loss[~ref["valid"]] == 0) and np.all(target[~ref["valid"]] == 0)


def test_split_depth_backward_is_deterministic(coda):
    wl = W.cross_entropy(seed=101, M=300, K=1024, V=1000, ignore_every=7)
    a, b = run_ce(coda, wl), run_ce(coda, wl)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    wl = W.swiglu_bwd(seed=102, M=333, Dm=1040, F=136)
    args = (to_dev_bf16(wl["dy"]), to_dev_bf16(wl["w_down"]), to_dev_bf16(wl["h"]))
    u = bf16_bits(coda.coda_gemm_swiglu_bwd_ws(*args))
    v = bf16_bits(coda.coda_gemm_swiglu_bwd_ws(*args))
    assert np.array_equal(u, v)


def test_no_split_equals_one_kernel_schedule_backward(coda):
    """Outputs of at least half as many tiles as CUs do not split: the *_ws entry points
    then run the one-kernel schedule, bit for bit."""
    M, K, V = 4096, 256, 4096
    assert coda.coda_split_workspace_bytes(M, V, K) == 0
    wl = W.cross_entropy(seed=103, M=M, K=K, V=V, ignore_every=11)
    for u, v in zip(run_ce(coda, wl), run_ce(coda, wl, split=False)):
        assert np.array_equal(u, v)
    M, Dm, F = 4096, 256, 4096
    assert coda.coda_split_workspace_bytes(M, F, Dm) == 0
    wl = W.swiglu_bwd(seed=104, M=M, Dm=Dm, F=F)
    args = (to_dev_bf16(wl["dy"]), to_dev_bf16(wl["w_down"]), to_dev_bf16(wl["h"]))
    assert np.array_equal(bf16_bits(coda.coda_gemm_swiglu_bwd_ws(*args)), bf16_bits(coda.coda_gemm_swiglu_bwd(*args)))


def test_split_depth_backward_workspace_errors(coda):
    import torch
    L = coda.lib()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    M, Dm, F = 333, 1040, 136
    need = coda.coda_split_workspace_bytes(M, F, Dm)
    dy = torch.zeros((M, Dm), dtype=torch.bfloat16, device="cuda")
    wd = torch.zeros((F, Dm), dtype=torch.bfloat16, device="cuda")
    h = torch.zeros((M, 2 * F), dtype=torch.bfloat16, device="cuda")
    dh = torch.empty((M, 2 * F), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    args = [p(dy), p(wd), p(h), M, Dm, F, p(dh)]
    assert L.coda_gemm_swiglu_bwd_ws(*args, p(ws), need - 16, None) == 4      # CODA_ERR_WORKSPACE
    assert L.coda_gemm_swiglu_bwd_ws(*args, None, 0, None) == 1               # CODA_ERR_NULL
    assert L.coda_gemm_swiglu_bwd_ws(*args, p(h), need, None) == 6            # workspace on an input
    assert L.coda_gemm_swiglu_bwd_ws(*args, p(ws), need, None) == 0
    M, K, V = 300, 1024, 1000
    need = coda.coda_split_workspace_bytes(M, V, K)
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((K, V), dtype=torch.bfloat16, device="cuda")
    labels = torch.zeros((M,), dtype=torch.int32, device="cuda")
    f = [torch.empty((M, coda.num_partials(V)), dtype=torch.float32, device="cuda")] + \
        [torch.empty((M,), dtype=torch.float32, device="cuda") for _ in range(3)]
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    args = [p(x), p(w), p(labels), M, K, V] + [p(t) for t in f]
    assert L.coda_gemm_cross_entropy_ws(*args, p(ws), need - 16, None) == 4
    assert L.coda_gemm_cross_entropy_ws(*args, p(f[0]), need, None) == 6       # workspace on an output
    assert L.coda_gemm_cross_entropy_ws(*args, p(ws), need, None) == 0
    sync()


def test_split_depth_replays_from_a_graph(coda):
    """The split-depth forward and SwiGLU backward captured in a HIP graph (two kernels
    per split GEMM, no memory set inside): each replay, with eager fills of the outputs
    and the workspace between replays, equals the eager call bit for bit."""
    import torch
    M, K, D, N1 = 300, 1024, 1032, 264
    wl = W.gemm_rmsnorm_fwd_inputs(105, M, K, D, N1, 1e-5)
    x, w0, z, g, w1 = (to_dev_bf16(wl[k]) for k in ("x", "w0", "z", "gamma", "w1"))
    outs = dict(h1=torch.empty((M, D), dtype=torch.bfloat16, device="cuda"),
                h2=torch.empty((M, D), dtype=torch.bfloat16, device="cuda"),
                partials=torch.empty((M, coda.num_partials(D)), dtype=torch.float32, device="cuda"),
                r=torch.empty((M,), dtype=torch.float32, device="cuda"),
                y=torch.empty((M, N1), dtype=torch.bfloat16, device="cuda"))
    ws = torch.empty((coda.coda_gemm_rmsnorm_fwd_workspace_bytes(M, K, D, N1),), dtype=torch.uint8, device="cuda")
    wb = W.swiglu_bwd(seed=106, M=333, Dm=1040, F=136)
    dy, wd, h = (to_dev_bf16(wb[k]) for k in ("dy", "w_down", "h"))
    dh = torch.empty((333, 272), dtype=torch.bfloat16, device="cuda")
    ws2 = torch.empty((coda.coda_split_workspace_bytes(333, 136, 1040),), dtype=torch.uint8, device="cuda")

    def run():
        coda.coda_gemm_rmsnorm_fwd_ws(x, w0, z, g, w1, wl["eps"], workspace=ws, **outs)
        coda.coda_gemm_swiglu_bwd_ws(dy, wd, h, dh=dh, workspace=ws2)

    def snapshot():
        return [bf16_bits(t) if t.dtype == torch.bfloat16 else t.cpu().numpy() for t in (*outs.values(), dh)]

    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        run()
    sync()
    want = snapshot()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    sync()
    for rep in range(3):
        for t in (*outs.values(), dh):
            t.fill_(0)
        ws.fill_(7)
        ws2.fill_(7)
        sync()
        graph.replay()
        sync()
        for a, b in zip(snapshot(), want):
            assert np.array_equal(a, b), f"replay {rep} differs from the eager call"


def test_calls_on_two_streams_overlap_safely(coda):
    """The library keeps no state between calls (each call's buffers are its own): the
    split forward and the split SwiGLU backward issued on two streams at once, from two
    host threads, equal the same calls made one after the other."""
    import threading
    import torch
    wl = W.gemm_rmsnorm_fwd_inputs(107, 300, 1024, 1032, 264, 1e-5)
    fwd_in = [to_dev_bf16(wl[k]) for k in ("x", "w0", "z", "gamma", "w1")]
    wb = W.swiglu_bwd(seed=108, M=333, Dm=1040, F=136)
    bwd_in = (to_dev_bf16(wb["dy"]), to_dev_bf16(wb["w_down"]), to_dev_bf16(wb["h"]))
    want_f = [bf16_bits(t) if t.dtype == torch.bfloat16 else t.cpu().numpy()
              for t in coda.coda_gemm_rmsnorm_fwd_ws(*fwd_in, wl["eps"])]
    want_b = bf16_bits(coda.coda_gemm_swiglu_bwd_ws(*bwd_in))
    sync()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = {}

    def run(i):
        with torch.cuda.stream(streams[i]):
            for rep in range(5):
                if i == 0:
                    got[(i, rep)] = coda.coda_gemm_rmsnorm_fwd_ws(*fwd_in, wl["eps"])
                else:
                    got[(i, rep)] = coda.coda_gemm_swiglu_bwd_ws(*bwd_in)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    sync()
    for rep in range(5):
        f = [bf16_bits(t) if t.dtype == torch.bfloat16 else t.cpu().numpy() for t in got[(0, rep)]]
        for a, b in zip(f, want_f):
            assert np.array_equal(a, b)
        assert np.array_equal(bf16_bits(got[(1, rep)]), want_b)


# ------------------------------------------------- the partial last wave of a larger output
def test_remainder_split_forward(coda):
    """GEMM2 with 384 tiles on 256 CUs: its full wave runs the one-kernel schedule and the
    128 tiles of the partial wave are split in 2 slices (64 steps each); every element
    against the oracle."""
    import torch
    M, K, D, N1 = 4096, 1024, 4096, 6144
    need = coda.coda_gemm_rmsnorm_fwd_workspace_bytes(M, K, D, N1)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert need == 128 * 2 * 256 * 1024
    log(f"remainder split fwd M={M} K={K} D={D} N1={N1}")
    wl = W.gemm_rmsnorm_fwd_inputs(109, M, K, D, N1, 1e-5)
    h1, h2, part, r, y = coda.coda_gemm_rmsnorm_fwd_ws(*(to_dev_bf16(wl[k]) for k in ("x", "w0", "z", "gamma", "w1")),
                                                       wl["eps"])
    sync()
    ref = O.gemm_rmsnorm_fwd(wl["x"], wl["w0"], wl["z"], wl["gamma"], wl["w1"], wl["eps"])
    assert_close_tiles("h1", dec(h1), ref["h1"])
    assert_close_tiles("r", r.cpu().numpy(), ref["r"], rel_fro=TIGHT)
    assert_close_tiles("y", dec(y), ref["y"])


def test_remainder_split_cross_entropy_and_nk(coda):
    """320 output tiles: 256 in the one-kernel schedule, the last 64 in 2 slices; a KN
    GEMM with the cross-entropy epilogue and an NK one with the SwiGLU backward map."""
    import torch
    M, K, V = 4096, 2048, 5120
    cus256 = torch.cuda.get_device_properties(0).multi_processor_count == 256
    assert not cus256 or coda.coda_split_workspace_bytes(M, V, K) == 64 * 2 * 256 * 1024
    log(f"remainder split cross_entropy M={M} K={K} V={V}")
    wl = W.cross_entropy(seed=110, M=M, K=K, V=V, ignore_every=13)
    loss, lse, target, tile = (t.cpu().numpy() for t in coda.coda_gemm_cross_entropy_ws(
        to_dev_bf16(wl["x"]), to_dev_bf16(wl["w"]), torch.from_numpy(wl["labels"]).cuda()))
    ref = O.gemm_cross_entropy(wl["x"], wl["w"], wl["labels"])
    assert_close_tiles("tile_lse", tile, ref["tile_lse"], rel_fro=TIGHT, tile_n=1)
    assert_close_tiles("loss", loss, ref["loss"], rel_fro=TIGHT)
    assert np.all(loss[~ref["valid"]] == 0) and np.all(target[~ref["valid"]] == 0)
    M, Dm, F = 4096, 2048, 5120
    assert not cus256 or coda.coda_split_workspace_bytes(M, F, Dm) == 64 * 2 * 256 * 1024
    log(f"remainder split swiglu_bwd M={M} Dm={Dm} F={F}")
    wb = W.swiglu_bwd(seed=111, M=M, Dm=Dm, F=F)
    args = (to_dev_bf16(wb["dy"]), to_dev_bf16(wb["w_down"]), to_dev_bf16(wb["h"]))
    dh = coda.coda_gemm_swiglu_bwd_ws(*args)
    one = coda.coda_gemm_swiglu_bwd(*args)
    sync()
    ref = O.gemm_swiglu_bwd(wb["dy"], wb["w_down"], wb["h"])["dh"]
    got = dec(dh)
    assert_close_tiles("dh", got, ref, tile_n=512)
    # the 256 tiles of the full wave are the one-kernel schedule's, bit for bit: at least
    # 256 / 320 of the elements (the split tiles' may also agree where the rounding does)
    same = bf16_bits(dh) == bf16_bits(one)
    assert not cus256 or same.mean() >= 256 / 320


def test_split_plan_matches_the_device(coda):
    """The host-side plan at the device's CU count asks for the workspace that the calls
    on this device ask for, all-split, remainder-split and one-kernel shapes alike."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for M, N, K in [(300, 264, 4096), (517, 392, 1064), (4096, 5120, 2048), (4096, 4096, 1024),
                    (8192, 4096, 14336), (1, 8, 8), (0, 256, 256), (40, 1 << 22, 8)]:
        s, steps, tile0, nbytes = coda.coda_split_plan(M, N, K, cus)
        log(f"split plan M={M} N={N} K={K} cus={cus}: S={s} steps={steps} tile0={tile0} bytes={nbytes}")
        assert nbytes == coda.coda_split_workspace_bytes(M, N, K)
        assert s >= 1 and (s == 1) == (nbytes == 0)
