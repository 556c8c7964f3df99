"""The decode step under HIP graph capture (GPU): kv_decode_step_noalloc
takes its workspace from the library's device array and issues no
allocation, copy, memset or synchronization, so a caller can capture it in a
graph and replay it. Captured once (after an eager call on the device, which
looks up the array's address), the graph is replayed four times, with new
queries written eagerly between replays; every replay's output and pool
image must equal kv_decode_step's, run eagerly on the same inputs, bit for
bit, and lie within 2e-3 of the oracle."""
import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-3

kv = None
orc = None


@pytest.fixture(scope="module", autouse=True)
def _setup():
    global kv, orc
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import __graft_entry__
    __graft_entry__.ensure_built()
    import oracle
    import paged_kv_cache_169_amd as k
    kv, orc = k, oracle
    yield


@pytest.mark.parametrize("q_len", [1, 4])
def test_noalloc_step_replays_in_a_graph(q_len):
    print(f"graph replay of the decode step, q_len {q_len}", flush=True)
    lens = [0, 15, 16, 47, 300, 1000, 129, 2047]
    c = wl.make_case(700 + q_len, len(lens), lens, 32, 8, 128, "bf16", pool_slack=1.2, device=DEV, append=q_len)
    pools = []
    for _ in range(2):
        p = kv.KVPool(c.num_blocks, c.n_kv, c.d, "bf16", device=DEV)
        p.K.copy_(c.K)
        p.V.copy_(c.V)
        pools.append(p)
    eager_pool, graph_pool = pools
    max_ctx = int(c.ctx_lens.max().item())
    q = c.q.clone()
    out_g = torch.full(tuple(q.shape), float("nan"), dtype=torch.float32, device=DEV)
    out_e = torch.full_like(out_g, float("nan"))
    nbytes = kv.paged_multi_token_attention_workspace_bytes(eager_pool, c.batch, c.n_h, q_len, max_ctx, kv.attn_opts())
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
    # eager call first: the device array's address is looked up outside capture
    kv.kv_decode_step_noalloc(graph_pool, c.k_new, c.v_new, q, out_g, c.tables, c.seq_lens, c.scale, max_ctx)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        kv.kv_decode_step_noalloc(graph_pool, c.k_new, c.v_new, q, out_g, c.tables, c.seq_lens, c.scale, max_ctx,
                                  stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    gen = torch.Generator(device=DEV).manual_seed(q_len)
    K_ref, V_ref = wl.to_host_bits(c.K), wl.to_host_bits(c.V)
    tab, sl = c.tables.cpu().numpy(), c.seq_lens.cpu().numpy()
    if q_len == 1:
        orc.append(K_ref, V_ref, wl.to_host_bits(c.k_new), wl.to_host_bits(c.v_new), tab, sl)
    else:
        kn, vn = wl.to_host_bits(c.k_new), wl.to_host_bits(c.v_new)
        for t in range(q_len):
            orc.append(K_ref, V_ref, np.ascontiguousarray(kn[:, t]), np.ascontiguousarray(vn[:, t]), tab, sl + t)
    for r in range(4):
        q.copy_(torch.randn(q.shape, generator=gen, device=DEV).to(torch.bfloat16))  # eager work between replays
        out_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        kv.kv_decode_step(eager_pool, c.k_new, c.v_new, q, out_e, c.tables, c.seq_lens, c.scale, max_ctx, ws)
        torch.cuda.synchronize()
        a, b = out_g.cpu().numpy(), out_e.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"replay {r}: output differs from the eager step"
        assert np.array_equal(graph_pool.blob.cpu().numpy(), eager_pool.blob.cpu().numpy()), f"replay {r}: pool differs"
        if q_len == 1:
            ref = orc.attention(K_ref, V_ref, wl.to_host_bits(q), tab, c.ctx_lens.cpu().numpy(), c.scale)
        else:
            ref = orc.attention_multi(K_ref, V_ref, wl.to_host_bits(q), tab, c.ctx_lens.cpu().numpy(), c.scale)
        assert float(np.max(np.abs(a.astype(np.float64) - ref))) <= TOL, f"replay {r}"
    del g
    for p in pools:
        p.close()
