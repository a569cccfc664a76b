"""The path captured in HIP graphs: the delayed-scaling step (fused amax+cast,
history update), the linear forward step, the per-block / grouped and MXFP8
paths, the re-quantising GEMM and the all-reduce parts.  Every replay must
match the same calls run eagerly, with eager work and synchronisations between
replays (graph memory nodes are not used by the path, and the cast's reduction
goes through a workspace, not cleared memory)."""

import numpy as np
import pytest
import torch

import fp8_precision_numerics_amd as fm
from gpu_helpers import announce, device

pytestmark = pytest.mark.gpu


def _state_arrays(st):
    return {k: getattr(st, k).detach().cpu().numpy().copy() for k in ("history", "head", "scale", "scale_inv", "amax", "sat")}


@pytest.mark.parametrize("fused", [False, True])
def test_graph_replays_match_eager_delayed_scaling(fused):
    """fused: the graph holds fp8_quantize_update (cast and history step in one
    call); the eager reference always runs the two separate calls."""
    dev = device()
    rng = np.random.default_rng(77)
    xs = [torch.from_numpy((rng.standard_normal((512, 1024)) * 3.0 ** t).astype(np.float32)).to(dev).to(torch.bfloat16)
          for t in range(4)]
    q_eager = torch.empty((512, 1024), dtype=torch.uint8, device=dev)
    q_graph = torch.empty_like(q_eager)
    eager = fm.DelayedScalingState("e4m3", 16, device=dev)
    st = fm.DelayedScalingState("e4m3", 16, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        warm = fm.DelayedScalingState("e4m3", 16, device=dev)
        warm.quantize(xs[0], q=q_graph, count_saturation=True)
        warm.update()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for x in xs:
            if fused:
                st.quantize_update(x, q=q_graph, count_saturation=True)
            else:
                st.quantize(x, q=q_graph, count_saturation=True)
                st.update()
    for replay in range(3):
        announce(f"graph replay {replay} fused={fused}")
        graph.replay()
        for x in xs:                       # the same four steps, eagerly
            eager.quantize(x, q=q_eager, count_saturation=True)
            eager.update()
        torch.cuda.synchronize()
        a, b = _state_arrays(st), _state_arrays(eager)
        for k in a:
            assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), (replay, k)
        assert torch.equal(q_graph, q_eager)
        # unrelated eager work on the stream between replays
        torch.zeros(1 << 20, device=dev).add_(1.0).sum().item()


def test_graph_replays_match_eager_linear_forward_step():
    """The forward step of a linear layer as the benchmark replays it: the cast
    of X, the cast-transpose of W (each with its history step) and the GEMM on
    the codes, captured once per input set and replayed alternately.  Every
    replay's codes, states and output must equal the same steps run eagerly."""
    dev = device()
    rng = np.random.default_rng(78)
    M, K, N = 384, 640, 528           # the cast-transpose wants multiples of 16
    sets = [(torch.from_numpy((rng.standard_normal((M, K)) * 2.0 ** j).astype(np.float32)).to(dev).to(torch.bfloat16),
             torch.from_numpy((rng.standard_normal((K, N)) * 0.02 * 3.0 ** j).astype(np.float32)).to(dev).to(torch.bfloat16))
            for j in range(2)]

    def make():
        return {"sx": fm.DelayedScalingState("e4m3", 16, device=dev), "sw": fm.DelayedScalingState("e4m3", 16, device=dev),
                "qx": torch.empty((M, K), dtype=torch.uint8, device=dev),
                "qw": torch.empty((N, K), dtype=torch.uint8, device=dev),
                "c": torch.empty((M, N), dtype=torch.bfloat16, device=dev)}

    def step(s, x, w):
        s["sx"].quantize_update(x, q=s["qx"])
        s["sw"].quantize_update(w, q_t=s["qw"])
        fm.fp8_gemm(s["qx"], "e4m3", s["qw"], "e4m3", s["sx"].scale_inv_used, s["sw"].scale_inv_used, s["c"])

    g, e = make(), make()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(make(), *sets[0])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for x, w in sets:
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            step(g, x, w)
        graphs.append(gr)
    for replay, j in enumerate([0, 1, 0, 1]):
        announce(f"linear forward step graph replay {replay} (input set {j})")
        graphs[j].replay()
        step(e, *sets[j])
        torch.cuda.synchronize()
        for k in ("sx", "sw"):
            a, b = _state_arrays(g[k]), _state_arrays(e[k])
            for f in a:
                assert np.array_equal(a[f].view(np.uint8), b[f].view(np.uint8)), (replay, k, f)
        for k in ("qx", "qw"):
            assert torch.equal(g[k], e[k]), (replay, k)
        assert torch.equal(g["c"].view(torch.int16), e["c"].view(torch.int16)), replay
        torch.zeros(1 << 20, device=dev).add_(1.0).sum().item()


@pytest.mark.parametrize("accum", ["exact", "mfma_fp8"])
def test_graph_replays_match_eager_blockwise_grouped_and_mx(accum):
    """The per-block quantisers and the grouped GEMM (three experts, one empty),
    the MXFP8 quantisers and the MXFP8 GEMM, captured in one graph: each of three
    replays, with eager work between them, must give the codes, scales and
    outputs of the same calls run eagerly, bit for bit."""
    dev = device()
    rng = np.random.default_rng(79)
    G, N, K, total = 3, 256, 384, 256
    offs = torch.tensor([0, 100, 100, total], dtype=torch.int32, device=dev)
    A = torch.from_numpy(rng.standard_normal((total, K)).astype(np.float32)).to(dev).to(torch.bfloat16)
    B = torch.from_numpy((rng.standard_normal((G * N, K)) * 0.02).astype(np.float32)).to(dev).to(torch.bfloat16)
    X = torch.from_numpy(rng.standard_normal((256, 256)).astype(np.float32)).to(dev)
    W = torch.from_numpy((rng.standard_normal((192, 256)) * 0.05).astype(np.float32)).to(dev)
    nkb = (K + 127) // 128

    def buffers():
        u8 = dict(dtype=torch.uint8, device=dev)
        return {"qa": torch.empty((total, K), **u8), "sa": torch.empty((total, nkb), device=dev),
                "qb": torch.empty((G * N, K), **u8), "sb": torch.empty((G * N // 128, nkb), device=dev),
                "c": torch.empty((total, N), device=dev),
                "qx": torch.empty((256, 256), **u8), "sx": torch.empty(8 * fm.mx_scale_ld(256), **u8),
                "qw": torch.empty((192, 256), **u8), "sw": torch.empty(8 * fm.mx_scale_ld(192), **u8),
                "cm": torch.empty((256, 192), device=dev)}

    def run(b):
        fm.fp8_quantize_blockwise(A, 1, "e4m3", b["qa"], b["sa"])
        fm.fp8_quantize_blockwise(B, 128, "e4m3", b["qb"], b["sb"])
        fm.fp8_grouped_gemm(b["qa"], b["sa"], b["qb"].view(G, N, K), b["sb"].view(G, N // 128, nkb), offs, b["c"],
                            accum=accum)
        fm.fp8_quantize_mx(X, "e4m3", b["qx"], b["sx"])
        fm.fp8_quantize_mx(W, "e4m3", b["qw"], b["sw"])
        fm.fp8_gemm_mx(b["qx"], "e4m3", b["sx"], b["qw"], "e4m3", b["sw"], b["cm"], accum=accum)

    g_buf, e_buf = buffers(), buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(g_buf)                                  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for t in g_buf.values():
        t.zero_()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(g_buf)
    for replay in range(3):
        announce(f"graph replay {replay} blockwise/grouped/mx {accum}")
        for t in e_buf.values():
            t.zero_()
        graph.replay()
        run(e_buf)
        torch.cuda.synchronize()
        for k in g_buf:
            a, b = g_buf[k], e_buf[k]
            if a.dtype == torch.float32:
                a, b = a.view(torch.int32), b.view(torch.int32)
            assert torch.equal(a, b), (replay, k)
        torch.zeros(1 << 20, device=dev).add_(1.0).sum().item()


@pytest.mark.parametrize("accum", ["exact", "mfma_fp8"])
def test_graph_replays_match_eager_requant_and_allreduce_parts(accum):
    """The GEMM with its output re-quantised in the epilogue (which clears and
    then accumulates its amax and count), and the all-reduce parts (shared scale
    over eight ranks' amaxes, cast of each rank's gradient with it, sum of the
    eight payloads), captured in one graph and replayed three times."""
    dev = device()
    rng = np.random.default_rng(80)
    M, N, K, R, n = 320, 272, 256, 8, 4096
    qa = torch.from_numpy(rng.integers(0, 0x7F, (M, K), dtype=np.uint8)).to(dev)
    qb = torch.from_numpy(rng.integers(0, 0x7F, (N, K), dtype=np.uint8)).to(dev)
    sa = torch.tensor([2.0 ** -9], device=dev)
    sb = torch.tensor([2.0 ** -8], device=dev)
    out_scale = torch.tensor([0.5], device=dev)
    grads = torch.from_numpy((rng.standard_normal((R, n)) * 1e-3).astype(np.float32)).to(dev)
    amaxes = grads.abs().amax(dim=1).contiguous()

    def buffers():
        return {"cq": torch.empty((M, N), dtype=torch.uint8, device=dev), "amax": torch.empty(1, device=dev),
                "sat": torch.empty(1, dtype=torch.int64, device=dev), "scale": torch.empty(1, device=dev),
                "scale_inv": torch.empty(1, device=dev), "q": torch.empty((R, n), dtype=torch.uint8, device=dev),
                "sum": torch.empty(n, device=dev)}

    def run(b):
        fm.fp8_gemm_requant(qa, "e4m3", qb, "e4m3", sa, sb, "e4m3", out_scale, b["cq"], amax=b["amax"],
                            sat=b["sat"], accum=accum)
        fm.fp8_shared_scale(amaxes, "e5m2", b["scale"], b["scale_inv"])
        for r in range(R):
            fm.fp8_quantize(grads[r], "e5m2", b["scale"], q=b["q"][r])
        fm.fp8_dequant_sum(b["q"], "e5m2", b["scale_inv"], b["sum"])

    g_buf, e_buf = buffers(), buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(g_buf)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(g_buf)
    for replay in range(3):
        announce(f"graph replay {replay} requant/allreduce {accum}")
        for t in list(g_buf.values()) + list(e_buf.values()):
            t.view(torch.uint8).fill_(0xA5)              # junk that every call must overwrite
        graph.replay()
        run(e_buf)
        torch.cuda.synchronize()
        for k in g_buf:
            assert torch.equal(g_buf[k].view(torch.uint8), e_buf[k].view(torch.uint8)), (replay, k)
        torch.zeros(1 << 20, device=dev).add_(1.0).sum().item()
