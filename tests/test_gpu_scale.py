"""Any finite softmax scale (GPU): the decode and multi-token kernels take
the scale as a caller argument ["KV Cache는 왜 LLM 서빙의 핵심인가",
section "KV Cache: O(T²)를 O(T)로": softmax(q K^T * scale)], and nothing
in them may assume its sign or size. Negative, zero and large scales run
through every tile engine (balanced and fixed-split MFMA, wide multi-token
units, INT4, VALU) against the oracle. Bound: max |error| <= 2e-3."""
import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-3
SCALES = [-0.3, 0.0, 2.0]
LENS = [0, 15, 16, 47, 300, 1000]

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


def check(got, ref):
    got = got.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - ref)))
    print(f"max |err| {err:.3g}", flush=True)
    assert err <= TOL


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("engine", ["balanced", "split", "valu"])
@pytest.mark.parametrize("g", [4, 16])
def test_decode_any_scale(scale, engine, g):
    print(f"decode scale={scale} engine={engine} g={g}", flush=True)
    c = wl.make_case(300 + g, len(LENS), LENS, 2 * g, 2, 128, "bf16", append=False, device=DEV)
    pool = kv.KVPool(c.num_blocks, c.n_kv, c.d, "bf16", device=DEV)
    pool.K.copy_(c.K)
    pool.V.copy_(c.V)
    opts = {"balanced": kv.attn_opts(kernel=2, schedule=0), "split": kv.attn_opts(kernel=2, schedule=1, split_blocks=3),
            "valu": kv.attn_opts(kernel=1, schedule=1)}[engine]
    max_ctx = int(c.ctx_lens.max().item())
    nbytes = kv.paged_decode_attention_workspace_bytes(pool, c.batch, c.n_h, max_ctx, opts)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
    out = torch.full((c.batch, c.n_h, c.d), float("nan"), dtype=torch.float32, device=DEV)
    kv.paged_decode_attention(pool, c.q, out, c.tables, c.ctx_lens, scale, max_ctx, ws, opts=opts)
    torch.cuda.synchronize()
    ref = orc.attention(wl.to_host_bits(c.K), wl.to_host_bits(c.V), wl.to_host_bits(c.q), c.tables.cpu().numpy(),
                        c.ctx_lens.cpu().numpy(), scale)
    check(out, ref)
    pool.close()


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("q_len", [3, 12, 40])
def test_multi_token_any_scale(scale, q_len):
    """4 query heads per kv head: 12, 48 and 160 query columns (one or two
    column tiles per unit, wide units of four and eight)."""
    print(f"multi-token scale={scale} q_len={q_len}", flush=True)
    c = wl.make_case(400 + q_len, len(LENS), [n + q_len for n in LENS], 8, 2, 128, "bf16", append=False, device=DEV)
    pool = kv.KVPool(c.num_blocks, c.n_kv, c.d, "bf16", device=DEV)
    pool.K.copy_(c.K)
    pool.V.copy_(c.V)
    g = torch.Generator(device=DEV).manual_seed(q_len)
    q = torch.randn((c.batch, q_len, c.n_h, c.d), generator=g, device=DEV).to(torch.bfloat16)
    opts = kv.attn_opts(kernel=2, schedule=0)
    max_ctx = int(c.ctx_lens.max().item())
    nbytes = kv.paged_multi_token_attention_workspace_bytes(pool, c.batch, c.n_h, q_len, max_ctx, opts)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
    out = torch.full((c.batch, q_len, c.n_h, c.d), float("nan"), dtype=torch.float32, device=DEV)
    kv.paged_multi_token_attention(pool, q, out, c.tables, c.ctx_lens, scale, max_ctx, ws, None, opts)
    torch.cuda.synchronize()
    ref = orc.attention_multi(wl.to_host_bits(c.K), wl.to_host_bits(c.V), wl.to_host_bits(q), c.tables.cpu().numpy(),
                              c.ctx_lens.cpu().numpy(), scale)
    check(out, ref)
    pool.close()


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("g", [4, 8])
def test_int4_any_scale(scale, g):
    """INT4 pool coded from bf16 (one score per lane at 4 query heads, the
    16-column path at 8) against the oracle on the dequantized values."""
    print(f"int4 scale={scale} g={g}", flush=True)
    B = len(LENS)
    c = wl.make_case(500 + g, B, LENS, 2 * g, 2, 128, "bf16", append=False, device=DEV)
    src = kv.KVPool(c.num_blocks, c.n_kv, c.d, "bf16", device=DEV)
    src.K.copy_(c.K)
    src.V.copy_(c.V)
    dst = kv.KVPool(c.num_blocks, c.n_kv, c.d, "int4", max_seqs=B, device=DEV)
    kv.kv_quantize_int4(dst, src, c.tables, c.ctx_lens)
    opts = kv.attn_opts(kernel=2, schedule=0)
    max_ctx = int(c.ctx_lens.max().item())
    nbytes = kv.paged_decode_attention_workspace_bytes(dst, B, c.n_h, max_ctx, opts)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
    out = torch.full((B, c.n_h, c.d), float("nan"), dtype=torch.float32, device=DEV)
    kv.paged_decode_attention(dst, c.q, out, c.tables, c.ctx_lens, scale, max_ctx, ws, opts=opts)
    torch.cuda.synchronize()
    img = orc.Q4Image(c.num_blocks, c.n_kv, c.d, B)
    tab, ctx = c.tables.cpu().numpy(), c.ctx_lens.cpu().numpy()
    orc.q4_quantize_pool(img, wl.to_host_bits(c.K), wl.to_host_bits(c.V), tab, ctx)
    Kd, Vd = orc.q4_dequant(img, tab, ctx)
    ref = orc.attention(Kd, Vd, wl.to_host_bits(c.q), tab, ctx, scale)
    check(out, ref)
    src.close()
    dst.close()
