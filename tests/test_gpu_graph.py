"""The entry points under HIP graph capture: the library allocates nothing and issues no memset,
so quantize + forward, and a split decode step, can be captured once and replayed.  Each replay,
with eager work and a synchronisation between replays, must equal the eager result bit for bit."""

import pytest

pytestmark = pytest.mark.gpu


def rand_bf16(shape, seed, scale=1.0):
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return (torch.randn(shape, device="cuda", generator=g) * scale).to(torch.bfloat16)


def test_quantize_and_forward_graph_replays():
    import torch
    from bit_attention_amd import ops
    B, H, N, d = 1, 4, 1024, 128
    q, k, v = rand_bf16((B, H, N, d), 1, 1.3), rand_bf16((B, H, N, d), 2), rand_bf16((B, H, N, d), 3)
    qc = torch.empty((B, H, N, d // 2), dtype=torch.uint8, device="cuda")
    qs = torch.empty((B, H, N, d // 32), dtype=torch.uint8, device="cuda")
    kc, ks = torch.empty_like(qc), torch.empty_like(qs)
    vc = torch.empty((B, H, N // 32, d, 16), dtype=torch.uint8, device="cuda")
    vs = torch.empty((B, H, N // 32, d), dtype=torch.uint8, device="cuda")
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    m = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    l = torch.empty_like(m)

    def step():
        ops.attn_fp4_quantize(q, 0, qc, qs)
        ops.attn_fp4_quantize(k, 0, kc, ks)
        ops.attn_fp4_quantize(v, 1, vc, vs)
        ops.attn_fp4_fwd(qc, qs, kc, ks, vc, vs, causal=True, o=o, m=m, l=l)

    step()
    torch.cuda.synchronize()
    ref = (o.clone(), m.clone(), l.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                   # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        o.zero_(); m.zero_(); l.zero_()          # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref[0]) and torch.equal(m, ref[1]) and torch.equal(l, ref[2]), r


def test_split_decode_graph_replays():
    import torch
    from bit_attention_amd import ops
    B, Hq, Hkv, Nk, d = 4, 8, 2, 2048, 128
    need = ops.attn_fp4_fwd_kvcache_workspace_bytes(B, Hq, Hkv, 1, Nk, d)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    q = rand_bf16((B, Hq, 1, d), 4, 1.3)
    kq = ops.attn_fp4_quantize(rand_bf16((B, Hkv, Nk, d), 5), 0)
    vq = ops.attn_fp4_quantize(rand_bf16((B, Hkv, Nk, d), 6), 1)
    qq = ops.attn_fp4_quantize(q, 0)
    sl = torch.tensor([2048, 1500, 7, 999], dtype=torch.int32, device="cuda")
    o = torch.empty((B, Hq, 1, d), dtype=torch.bfloat16, device="cuda")
    m = torch.empty((B, Hq, 1), dtype=torch.float32, device="cuda")
    l = torch.empty_like(m)
    step = lambda: ops.attn_fp4_fwd_kvcache(*qq, *kq, *vq, seqlens_k=sl, causal=True, o=o, m=m, l=l, workspace=ws)
    step()
    torch.cuda.synchronize()
    ref = (o.clone(), m.clone(), l.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        o.zero_(); ws.zero_()                    # stale workspace contents must not matter
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref[0]) and torch.equal(m, ref[1]) and torch.equal(l, ref[2]), r


def test_nvfp4_quantize_and_forward_graph_replays():
    # the tensor amax is cleared by a kernel, not a memset, so the NVFP4-style path captures too
    import torch
    from bit_attention_amd import ops
    B, Hq, Hkv, N, d = 1, 4, 2, 512, 128
    q, k, v = rand_bf16((B, Hq, N, d), 7, 1.3), rand_bf16((B, Hkv, N, d), 8), rand_bf16((B, Hkv, N, d), 9)
    qq, kq, vq = ops.attn_fp4_nv_quantize(q, 0), ops.attn_fp4_nv_quantize(k, 0), ops.attn_fp4_nv_quantize(v, 1)
    ws = torch.empty(ops.attn_fp4_nv_fwd_workspace_bytes(B, Hq, Hkv, N, d), dtype=torch.uint8, device="cuda")
    o = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device="cuda")
    m = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")
    l = torch.empty_like(m)

    def step():
        for x, axis, out in ((q, 0, qq), (k, 0, kq), (v, 1, vq)):
            ops.attn_fp4_nv_quantize(x, axis, *out)
        ops.attn_fp4_nv_fwd(*qq, *kq, *vq, causal=True, o=o, m=m, l=l, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = (o.clone(), m.clone(), l.clone(), qq[2].clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(3):
        o.zero_(); m.zero_(); l.zero_(); ws.zero_(); qq[2].fill_(7.0)   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref[0]) and torch.equal(m, ref[1]) and torch.equal(l, ref[2]), r
        assert torch.equal(qq[2], ref[3]), r
