"""The prefill steps captured in a HIP graph and replayed: NVFP4 (quantize X,
quantize W with dynamic tensor scales, W4A4 GEMM on 256x320 tiles at the
4096 x 10240 x 5120 shape) and MXFP4 (balance-scaled Hadamard quantization
of X and W, W4A4 GEMM at 2048 x 14336 x 4096).  Every replay, with the
static inputs changed and eager library calls in between, must give the
same bits as the eager step on the same inputs."""
import pytest
import torch

from gpu_util import fp4q

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(seed, m, n, k):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    x = torch.randn(m, k, device=DEV, generator=g)
    x[:, torch.randperm(k, device=DEV, generator=g)[:8]] *= 40.0      # outlier channels
    w = torch.randn(n, k, device=DEV, generator=g) * 0.02
    return x.to(torch.bfloat16), w.to(torch.bfloat16)


def _replays(step, static, variants):
    """Eager results for each input set, then graph replays that cycle
    through the sets; returns after checking every replay."""
    L = fp4q()
    want = []
    for xv, wv in variants:
        static[0].copy_(xv)
        static[1].copy_(wv)
        want.append(step().clone())
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = step()
    for i in range(2 * len(variants)):
        v = i % len(variants)
        static[0].copy_(variants[v][0])
        static[1].copy_(variants[v][1])
        print(f"replay {i} (input set {v})", flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want[v]), f"replay {i} differs from the eager step"
        # eager library work between replays, on another shape
        y = L.gemm_w4a4(L.NVFP4, *L.quantize_nvfp4(variants[0][0][:256]), *L.quantize_nvfp4(variants[0][1][:384]))
        torch.cuda.synchronize()
        assert torch.isfinite(y).all()


def test_nvfp4_prefill_step_graph_replays():
    L = fp4q()
    m, n, k = 4096, 10240, 5120
    variants = [_inputs(700, m, n, k), _inputs(701, m, n, k)]
    variants[1] = (variants[1][0] * 3.0, variants[1][1])             # another tensor scale
    x = variants[0][0].clone()
    w = variants[0][1].clone()
    xq = (torch.empty((m, k // 2), dtype=torch.uint8, device=DEV),
          torch.empty((m, k // 16), dtype=torch.uint8, device=DEV),
          torch.empty(1, dtype=torch.float32, device=DEV))
    wq = (torch.empty((n, k // 2), dtype=torch.uint8, device=DEV),
          torch.empty((n, k // 16), dtype=torch.uint8, device=DEV),
          torch.empty(1, dtype=torch.float32, device=DEV))
    y = torch.empty((m, n), dtype=torch.float32, device=DEV)

    def step():
        L.quantize_nvfp4(x, out=xq)
        L.quantize_nvfp4(w, out=wq)
        L.gemm_w4a4(L.NVFP4, *xq, *wq, out=y)
        return y

    print("NVFP4 step 4096 x 10240 x 5120 under graph capture", flush=True)
    _replays(step, (x, w), variants)


def test_mxfp4_prefill_step_graph_replays():
    L = fp4q()
    m, n, k = 2048, 14336, 4096
    variants = [_inputs(702, m, n, k), _inputs(703, m, n, k)]
    x = variants[0][0].clone()
    w = variants[0][1].clone()
    t = torch.rand(k, device=DEV, generator=torch.Generator(device=DEV).manual_seed(704)) + 0.5
    u = 1.0 / t
    y = torch.empty((m, n), dtype=torch.float32, device=DEV)
    xq = (torch.empty((m, k // 2), dtype=torch.uint8, device=DEV), torch.empty((m, k // 32), dtype=torch.uint8, device=DEV))
    wq = (torch.empty((n, k // 2), dtype=torch.uint8, device=DEV), torch.empty((n, k // 32), dtype=torch.uint8, device=DEV))

    def step():
        L.quantize_mxfp4(x, t, True, out=xq)
        L.quantize_mxfp4(w, u, True, out=wq)
        L.gemm_w4a4(L.MXFP4, xq[0], xq[1], None, wq[0], wq[1], None, out=y)
        return y

    print("MXFP4 step 2048 x 14336 x 4096 under graph capture", flush=True)
    _replays(step, (x, w), variants)
