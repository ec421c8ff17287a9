"""Every entry point can be captured in a HIP graph: a replay writes the
same bytes as the eager call, on every replay, with eager calls and other
device work between the replays (the library allocates nothing and records
no memset, so a captured call is just its kernels)."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


def G():
    import gemm_wq_quantize_amd as g
    return g


def replay_matches_eager(launch, out, other):
    """launch(out) enqueues one call writing ``out`` (a tensor or a tuple of
    tensors); ``other`` has the same shapes and is written by eager calls
    between the replays."""
    outs = out if isinstance(out, tuple) else (out,)
    launch(out)
    torch.cuda.synchronize()
    refs = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            launch(out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    others = other if isinstance(other, tuple) else (other,)
    for i in range(4):
        for t in outs:
            t.view(torch.uint8).fill_(0xA5)    # poison: the replay must rewrite every byte
        launch(other)                          # eager work between replays
        torch.randn(1 << 20, device="cuda").sum()
        graph.replay()
        torch.cuda.synchronize()
        for t, o, r in zip(outs, others, refs):
            assert torch.equal(t.view(torch.uint8), r.view(torch.uint8)), f"replay {i}"
            assert torch.equal(o.view(torch.uint8), r.view(torch.uint8)), f"eager {i}"


def rand_codes(n, k, gen):
    return torch.randint(0, 16, (n, k), dtype=torch.uint8, generator=gen).cuda()


@pytest.mark.parametrize("c", [1, 2, 4, 8, 16, 32])
def test_graph_gemv_w4(c):
    say("graph wq_gemv_w4", c)
    g = G()
    gen = torch.Generator().manual_seed(c)
    k, n = 5120, 4096
    pk = torch.empty((n, k // 2), dtype=torch.uint8, device="cuda")
    g.wq_pack_int4(rand_codes(n, k, gen), g.LAYOUT_GFX950, pk)
    sc = (0.002 + 0.018 * torch.rand((n, k // 128), generator=gen)).bfloat16().cuda()
    x = torch.randn((c, k), generator=gen).bfloat16().cuda()
    out = torch.empty((c, n), dtype=torch.bfloat16, device="cuda")
    other = torch.empty_like(out)
    replay_matches_eager(lambda o: g.wq_gemv_w4(pk, g.LAYOUT_GFX950, sc, None, 8.0, k, 128, x, o), out, other)


@pytest.mark.parametrize("group", [128, 1024])
def test_graph_gemm_w4a16(group):
    say("graph wq_gemm_w4a16", group)
    g = G()
    gen = torch.Generator().manual_seed(group)
    m, n, k = 320, 640, 1024
    b = torch.empty((n, k // 2), dtype=torch.uint8, device="cuda")
    g.wq_pack_int4(rand_codes(n, k, gen), g.LAYOUT_GFX950, b)
    a = torch.randn((m, k), generator=gen).bfloat16().cuda()
    sc = (0.002 + 0.018 * torch.rand((n, k // group), generator=gen)).bfloat16().cuda()
    out = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    other = torch.empty_like(out)
    replay_matches_eager(lambda o: g.wq_gemm_w4a16(a, b, g.LAYOUT_GFX950, sc, group, 8.0, o), out, other)


def test_graph_quantize_pack_int4():
    say("graph wq_quantize_pack_int4")
    g = G()
    gen = torch.Generator().manual_seed(5)
    n, k = 1024, 4096
    w = (0.02 * torch.randn((n, k), generator=gen)).half().cuda()
    bufs = [(torch.empty((n, k // 2), dtype=torch.uint8, device="cuda"),
             torch.empty((n, k // 128), dtype=torch.bfloat16, device="cuda")) for _ in range(2)]
    replay_matches_eager(lambda o: g.wq_quantize_pack_int4(w, 128, g.LAYOUT_GFX950, o[0], o[1]),
                         bufs[0], bufs[1])


@pytest.mark.parametrize("c", [1, 4, 8, 64])
def test_graph_gemv_ternary(c):
    say("graph wq_gemv_ternary", c)
    g = G()
    gen = torch.Generator().manual_seed(100 + c)
    n, k = 4000, 5120
    trits = torch.randint(-1, 2, (n, k), dtype=torch.int8, generator=gen).cuda()
    d = (0.01 + 0.04 * torch.rand((n, k // 128), generator=gen)).half().cuda()
    wb = torch.empty((n, k // 128, 28), dtype=torch.uint8, device="cuda")
    g.wq_pack_ptq1_0(trits, d, wb)
    xq = torch.empty((c, k // 32, 36), dtype=torch.uint8, device="cuda")
    g.wq_quantize_q8_1(torch.randn((c, k), generator=gen).cuda(), xq)
    out = torch.empty((c, n), dtype=torch.float32, device="cuda")
    other = torch.empty_like(out)
    replay_matches_eager(lambda o: g.wq_gemv_ternary(wb, xq, k, o), out, other)


def test_graph_pack_and_q8_1():
    say("graph wq_pack_ptq1_0 / wq_quantize_q8_1 / wq_pack_int4")
    g = G()
    gen = torch.Generator().manual_seed(7)
    n, k = 300, 1024
    trits = torch.randint(-1, 2, (n, k), dtype=torch.int8, generator=gen).cuda()
    d = (0.01 + 0.04 * torch.rand((n, k // 128), generator=gen)).half().cuda()
    wb, wb2 = (torch.empty((n, k // 128, 28), dtype=torch.uint8, device="cuda") for _ in range(2))
    replay_matches_eager(lambda o: g.wq_pack_ptq1_0(trits, d, o), wb, wb2)
    x = torch.randn((5, k), generator=gen).cuda()
    xq, xq2 = (torch.empty((5, k // 32, 36), dtype=torch.uint8, device="cuda") for _ in range(2))
    replay_matches_eager(lambda o: g.wq_quantize_q8_1(x, o), xq, xq2)
    codes = rand_codes(n, k, gen)
    pk, pk2 = (torch.empty((n, k // 2), dtype=torch.uint8, device="cuda") for _ in range(2))
    replay_matches_eager(lambda o: g.wq_pack_int4(codes, g.LAYOUT_GFX950, o), pk, pk2)


def _ternary_operands(n, k, c, gen):
    g = G()
    trits = torch.randint(-1, 2, (n, k), dtype=torch.int8, generator=gen).cuda()
    d = (0.01 + 0.04 * torch.rand((n, k // 128), generator=gen)).half().cuda()
    wb = torch.empty((n, k // 128, 28), dtype=torch.uint8, device="cuda")
    g.wq_pack_ptq1_0(trits, d, wb)
    x = torch.randn((c, k), generator=gen).cuda()
    return wb, x


@pytest.mark.parametrize("c", [1, 4, 64])
def test_graph_ternary_pt_layout(c):
    say("graph wq_quantize_q8_1_pt / wq_gemv_ternary_pt", c)
    g = G()
    gen = torch.Generator().manual_seed(200 + c)
    n, k = 2000, 5120
    wb, x = _ternary_operands(n, k, c, gen)
    xp, xp2 = (torch.empty((c, 9 * k // 8), dtype=torch.uint8, device="cuda") for _ in range(2))
    replay_matches_eager(lambda o: g.wq_quantize_q8_1_pt(x, o), xp, xp2)
    out = torch.empty((c, n), dtype=torch.float32, device="cuda")
    replay_matches_eager(lambda o: g.wq_gemv_ternary_pt(wb, xp, k, o), out, torch.empty_like(out))


@pytest.mark.parametrize("c", [1, 8, 64])
def test_graph_gemv_ternary_ptq1_1(c):
    say("graph wq_gemv_ternary_ptq1_1 / _pt", c)
    g = G()
    gen = torch.Generator().manual_seed(300 + c)
    n, k = 1000, 5120
    wb, x = _ternary_operands(n, k, c, gen)
    sup, book, ei, ep = (torch.from_numpy(a).cuda() for a in g.wq_ptq1_1_encode(wb.cpu().numpy()))
    xq = torch.empty((c, k // 32, 36), dtype=torch.uint8, device="cuda")
    g.wq_quantize_q8_1(x, xq)
    xp = torch.empty((c, 9 * k // 8), dtype=torch.uint8, device="cuda")
    g.wq_quantize_q8_1_pt(x, xp)
    out = torch.empty((c, n), dtype=torch.float32, device="cuda")
    replay_matches_eager(lambda o: g.wq_gemv_ternary_ptq1_1(sup, book, ei, ep, xq, k, o), out, torch.empty_like(out))
    replay_matches_eager(lambda o: g.wq_gemv_ternary_ptq1_1_pt(sup, book, ei, ep, xp, k, o), out,
                         torch.empty_like(out))


def test_graph_gemv_ternary_noalloc():
    say("graph wq_gemv_ternary_noalloc", 64)
    g = G()
    gen = torch.Generator().manual_seed(400)
    n, k, c = 1000, 5120, 64
    wb, x = _ternary_operands(n, k, c, gen)
    xq = torch.empty((c, k // 32, 36), dtype=torch.uint8, device="cuda")
    g.wq_quantize_q8_1(x, xq)
    out = torch.empty((c, n), dtype=torch.float32, device="cuda")
    replay_matches_eager(lambda o: g.wq_gemv_ternary_noalloc(wb, xq, k, o), out, torch.empty_like(out))
