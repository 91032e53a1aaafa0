"""fp8_quantize (both of its paths), a product, a split product and an
accumulating product captured as HIP graphs: every replay, with the inputs
rewritten in place and eager work between the replays, gives the eager
calls' outputs bit for bit.  The library launches on
torch's current stream, so capture records its kernels (no memset nodes: the
amax word is cleared by a kernel)."""
import pytest
import torch

from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fl():
    return need_gpu()


@pytest.mark.parametrize("n_rows", [96, 4096])   # 48 KiB (one workgroup) and 2 MiB (three launches) of bf16 x
def test_quantize_and_product_replayed_from_a_graph(fl, n_rows):
    K, N = 256, 192
    g = torch.Generator(device="cuda").manual_seed(n_rows)
    x = torch.empty(n_rows, K, dtype=torch.bfloat16, device="cuda")
    w = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    x8 = torch.empty(n_rows, K, dtype=torch.uint8, device="cuda")
    w8 = torch.empty(N, K, dtype=torch.uint8, device="cuda")
    bx, bw = (torch.empty(1, dtype=torch.int32, device="cuda") for _ in range(2))
    ax, aw = (torch.empty(1, dtype=torch.float32, device="cuda") for _ in range(2))
    y = torch.empty(n_rows, N, dtype=torch.float32, device="cuda")

    def step():
        fl.quantize(x, fl.E4M3, 0, out=x8, bias=bx, amax=ax)
        fl.quantize(w, fl.E4M3, 1, out=w8, bias=bw, amax=aw)
        fl.scaled_gemm_fwd(x8, fl.E4M3, bx, w8, fl.E4M3, bw, out=y)

    def outputs():
        return [t.clone() for t in (x8, w8, bx, bw, ax.view(torch.int32), aw.view(torch.int32), y.view(torch.int32))]

    def fill(seed):
        x.copy_((torch.randn(n_rows, K, device="cuda", generator=torch.Generator(device="cuda").manual_seed(seed))
                 * (1 + seed)).to(torch.bfloat16))

    fill(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    for r in range(4):
        say("graph replay", "rows", n_rows, "replay", r)
        fill(r + 1)
        step()                      # eager reference for this input
        torch.cuda.synchronize()
        ref = outputs()
        for t in (x8, w8, bx, bw, ax, aw, y):   # clobber what the replay must rewrite
            t.fill_(7)
        graph.replay()
        torch.cuda.synchronize()
        got = outputs()
        for i, (a, b) in enumerate(zip(ref, got)):
            assert torch.equal(a, b), (n_rows, r, i)


def test_split_product_replayed_from_a_graph(fl):
    """A product split along the contraction (its two kernels: slices, then
    the ordered sum) captured as a graph: every replay, with new operands
    written in place and eager calls between, equals the eager call bit for bit."""
    M, N, K = 128, 1024, 4096
    nbytes = fl.gemm_workspace_bytes(fl.OP_FWD, M, N, K)
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    x = torch.empty(M, K, dtype=torch.bfloat16, device="cuda")
    w = (torch.randn(N, K, device="cuda", generator=torch.Generator(device="cuda").manual_seed(3)) * 0.02).to(torch.bfloat16)
    x8 = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    w8 = torch.empty(N, K, dtype=torch.uint8, device="cuda")
    bx, bw = (torch.empty(1, dtype=torch.int32, device="cuda") for _ in range(2))
    ax, aw = (torch.empty(1, dtype=torch.float32, device="cuda") for _ in range(2))
    y = torch.empty(M, N, dtype=torch.float32, device="cuda")

    def step():
        fl.quantize(x, fl.E4M3, 0, out=x8, bias=bx, amax=ax)
        fl.quantize(w, fl.E4M3, 0, out=w8, bias=bw, amax=aw)
        fl.scaled_gemm(fl.OP_FWD, x8, fl.E4M3, bx, w8, fl.E4M3, bw, out=y, workspace=ws)

    def fill(seed):
        g = torch.Generator(device="cuda").manual_seed(100 + seed)
        x.copy_((torch.randn(M, K, device="cuda", generator=g) * (1 + seed)).to(torch.bfloat16))

    fill(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    for r in range(4):
        say("graph replay, split product", "replay", r)
        fill(r + 1)
        step()
        torch.cuda.synchronize()
        ref = y.clone()
        y.fill_(7)
        ws.fill_(7)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ref.view(torch.int32), y.view(torch.int32)), r



def test_accumulating_product_replayed_from_a_graph(fl):
    """fp8_scaled_gemm_accumulate captured as a graph (a weight gradient summed
    over micro-batches): each replay adds the product of the operands then in
    place to the buffer.  A replay from a given buffer equals the eager call
    from the same buffer bit for bit, and so does a second replay on top of
    the first."""
    M, N, K = 1024, 768, 512    # wgrad: dY8 [M x N], X8 [M x K] -> dW [N x K]
    dy8 = torch.empty(M, N, dtype=torch.uint8, device="cuda")
    x8 = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    bdy = torch.tensor([20], dtype=torch.int32, device="cuda")
    bx = torch.tensor([3], dtype=torch.int32, device="cuda")
    dw = torch.zeros(N, K, dtype=torch.float32, device="cuda")

    def codes(t, seed, dtype):
        v = torch.randn(t.shape, device="cuda", generator=torch.Generator(device="cuda").manual_seed(seed))
        t.copy_((v * 8).to(dtype).view(torch.uint8))

    def step():
        fl.scaled_gemm_accumulate(fl.OP_WGRAD, dy8, fl.E5M2, bdy, x8, fl.E4M3, bx, dw)

    codes(dy8, 1, torch.float8_e5m2)
    codes(x8, 2, torch.float8_e4m3fn)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step()
    for r in range(4):
        say("graph replay, accumulating product", "replay", r)
        codes(x8, 10 + r, torch.float8_e4m3fn)
        start = dw.clone()
        step()                          # eager: start + product
        torch.cuda.synchronize()
        ref1 = dw.clone()
        dw.copy_(start)
        graph.replay()                  # the same from the same buffer
        torch.cuda.synchronize()
        assert torch.equal(ref1.view(torch.int32), dw.view(torch.int32)), r
        graph.replay()                  # a second product on top
        torch.cuda.synchronize()
        got2 = dw.clone()
        dw.copy_(ref1)
        step()                          # eager from the same buffer
        torch.cuda.synchronize()
        assert torch.equal(got2.view(torch.int32), dw.view(torch.int32)), r
        assert not torch.equal(got2, ref1)
