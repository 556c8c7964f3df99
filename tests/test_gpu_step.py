"""kv_decode_step (append then attend in one call) against the two calls it
stands for: kv_append_tokens, then paged_multi_token_attention over the
lengths after the append. On bf16 pools the append is fused into the MFMA
attention kernel; the pools and the outputs must still be bit-identical to
the separate calls (the same arithmetic on the same bits). One case also goes
to the oracle directly.
"""
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


def pools_for(c, dtype):
    """Two identical pools (INT4: coded from the case's bf16 cache)."""
    out = []
    for _ in range(2):
        if dtype == "int4":
            src = kv.KVPool(c.num_blocks, c.n_kv, c.d, "bf16", device=DEV)
            src.K.copy_(c.K)
            src.V.copy_(c.V)
            p = kv.KVPool(c.num_blocks, c.n_kv, c.d, "int4", max_seqs=c.batch, device=DEV)
            p.blob.zero_()  # tail rows the coder leaves alone must start equal in both pools
            kv.kv_quantize_int4(p, src, c.tables, c.seq_lens)
        else:
            p = kv.KVPool(c.num_blocks, c.n_kv, c.d, dtype, device=DEV)
            p.K.copy_(c.K)
            p.V.copy_(c.V)
        out.append(p)
    return out


def region_bytes(pool):
    torch.cuda.synchronize()
    return pool.blob.cpu().numpy().copy()


def run_both(c, dtype, q_len, split=0, window=0, seq_lens=None, tables=None):
    seq_lens = c.seq_lens if seq_lens is None else seq_lens
    tables = c.tables if tables is None else tables
    ctx = seq_lens + q_len
    max_ctx = int(c.ctx_lens.max().item())
    pa, pb = pools_for(c, dtype)
    opts = kv.attn_opts(split_blocks=split, window=window)
    nbytes = kv.paged_multi_token_attention_workspace_bytes(pa, c.batch, c.n_h, q_len, max_ctx, opts)
    ws_a = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
    ws_b = torch.empty_like(ws_a)
    q = c.q
    out_a = torch.full(q.shape, 7.0, dtype=torch.float32, device=DEV)
    out_b = torch.full(q.shape, 7.0, dtype=torch.float32, device=DEV)
    slots = torch.arange(c.batch, dtype=torch.int32, device=DEV)
    # separate calls
    if q_len == 1:
        kv.kv_append(pa, c.k_new, c.v_new, tables, seq_lens, seq_slots=slots)
    else:
        kv.kv_append_tokens(pa, c.k_new, c.v_new, tables, seq_lens, seq_slots=slots)
    if q_len == 1:
        kv.paged_decode_attention(pa, q, out_a, tables, ctx, c.scale, max_ctx, ws_a, seq_slots=slots, opts=opts)
    else:
        kv.paged_multi_token_attention(pa, q, out_a, tables, ctx, c.scale, max_ctx, ws_a, seq_slots=slots, opts=opts)
    # one step
    kv.kv_decode_step(pb, c.k_new, c.v_new, q, out_b, tables, seq_lens, c.scale, max_ctx, ws_b, seq_slots=slots,
                      opts=opts)
    torch.cuda.synchronize()
    return pa, pb, out_a, out_b


def assert_same(pa, pb, out_a, out_b):
    assert np.array_equal(region_bytes(pa), region_bytes(pb)), "pool contents differ"
    a, b = out_a.cpu().numpy(), out_b.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"outputs differ: max {np.nanmax(np.abs(a - b))}"


CASES = [  # n_h, n_kv, d, lens
    (32, 8, 128, [511, 512, 95, 1000, 16, 0, 33, 2047]),
    (8, 2, 64, [37, 50, 15, 31, 64, 1]),
    (64, 8, 128, [300, 129, 7]),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("q_len", [1, 3, 16])
@pytest.mark.parametrize("split,window", [(0, 0), (2, 0), (0, 37), (3, 40)])
def test_step_bf16_fused_matches_separate_calls(case, q_len, split, window):
    n_h, n_kv, d, lens = CASES[case]
    print(f"step bf16 case={case} q_len={q_len} split={split} window={window}", flush=True)
    c = wl.make_case(40 + case, len(lens), lens, n_h, n_kv, d, "bf16", pool_slack=1.2, device=DEV, append=q_len)
    assert_same(*run_both(c, "bf16", q_len, split, window))


INT4_LENS = [  # lengths before the step: the new token starts a block, fills one (slot 15), or lands inside
    [100, 16, 47, 400, 3],
    [15, 31, 0, 255, 1023, 64, 17, 2047],
]


@pytest.mark.parametrize("lens", range(len(INT4_LENS)))
@pytest.mark.parametrize("q_len", [1, 5])
@pytest.mark.parametrize("split,window", [(0, 0), (2, 0), (0, 40)])
def test_step_int4_matches_separate_calls(lens, q_len, split, window):
    """INT4 with one new token: the append is fused into the attention kernel
    (coding in the workgroup that reads the last block); with 5 the append
    kernel runs first. Pools and outputs bit-identical to the separate calls."""
    print(f"step int4 lens={lens} q_len={q_len} split={split} window={window}", flush=True)
    ls = INT4_LENS[lens]
    c = wl.make_case(50 + lens, len(ls), ls, 32, 8, 128, "bf16", pool_slack=1.2, device=DEV, append=q_len,
                     outliers=4)
    assert_same(*run_both(c, "int4", q_len, split, window))


def test_step_int4_bad_rows():
    """INT4 fused step: a negative length and an out-of-range block id give NaN
    rows and leave the pool as the separate calls leave it."""
    lens = [100, 60, 200, 31]
    c = wl.make_case(54, 4, lens, 32, 8, 128, "bf16", pool_slack=1.2, device=DEV, append=True)
    seq_lens = c.seq_lens.clone()
    seq_lens[1] = -1
    tables = c.tables.clone()
    tables[2, 200 // 16] = -7
    pa, pb, out_a, out_b = run_both(c, "int4", 1, seq_lens=seq_lens, tables=tables)
    assert np.array_equal(region_bytes(pa), region_bytes(pb)), "pool contents differ"
    o = out_b.cpu().numpy()
    assert np.all(np.isnan(o[1])) and np.all(np.isnan(o[2]))
    a = out_a.cpu().numpy()
    keep = [0, 3]
    assert np.array_equal(a[keep].view(np.uint32), o[keep].view(np.uint32))


@pytest.mark.parametrize("split", [0, 2])
def test_step_int4_bad_block_before_the_last(split):
    """INT4 fused step with an out-of-range block id before a sequence's last
    block: that sequence's rows are NaN, its new token is still coded into
    its (valid) last block as the append kernel codes it, and the pools
    match the separate calls byte for byte."""
    lens = [100, 60, 200, 31]
    c = wl.make_case(55 + split, 4, lens, 32, 8, 128, "bf16", pool_slack=1.2, device=DEV, append=True)
    tables = c.tables.clone()
    tables[0, 5] = -7            # block 5 of 7; the token goes to block 6
    tables[2, 0] = 1 << 30       # the first block; the token goes to block 12
    pa, pb, out_a, out_b = run_both(c, "int4", 1, split, tables=tables)
    assert np.array_equal(region_bytes(pa), region_bytes(pb)), "pool contents differ"
    o = out_b.cpu().numpy()
    assert np.all(np.isnan(o[0])) and np.all(np.isnan(o[2]))
    a = out_a.cpu().numpy()
    keep = [1, 3]
    assert np.array_equal(a[keep].view(np.uint32), o[keep].view(np.uint32))


@pytest.mark.parametrize("split", [0, 1])
def test_step_f32_composed_matches_separate_calls(split):
    c = wl.make_case(51, 4, [37, 50, 16, 0], 4, 2, 64, "f32", pool_slack=1.3, device=DEV, append=True)
    assert_same(*run_both(c, "f32", 1, split))


def test_step_bad_rows():
    """A negative length, and a new token whose block id is out of range: the
    row reads NaN, nothing is written for it, other rows are unaffected."""
    lens = [100, 60, 200, 31]
    c = wl.make_case(52, 4, lens, 32, 8, 128, "bf16", pool_slack=1.2, device=DEV, append=True)
    seq_lens = c.seq_lens.clone()
    seq_lens[1] = -1
    tables = c.tables.clone()
    tables[2, 200 // 16] = -7
    pa, pb, out_a, out_b = run_both(c, "bf16", 1, seq_lens=seq_lens, tables=tables)
    assert np.array_equal(region_bytes(pa), region_bytes(pb)), "pool contents differ"
    o = out_b.cpu().numpy()
    # row 1: the separate calls see length -1 + 1 = 0 (an empty sequence, output
    # 0); the step sees the negative length before the append and reports it
    assert np.all(np.isnan(o[1])) and np.all(np.isnan(o[2]))
    assert np.all(np.isfinite(o[[0, 3]]))
    a = out_a.cpu().numpy()
    keep = [0, 2, 3]
    assert np.array_equal(np.isnan(a[keep]), np.isnan(o[keep]))
    assert np.array_equal(np.nan_to_num(a[keep]), np.nan_to_num(o[keep]))


def test_step_against_oracle():
    c = wl.make_case(53, 6, [5, 16, 17, 250, 1023, 64], 16, 4, 128, "bf16", pool_slack=1.2, device=DEV, append=4)
    pool = kv.KVPool(c.num_blocks, c.n_kv, c.d, "bf16", device=DEV)
    pool.K.copy_(c.K)
    pool.V.copy_(c.V)
    max_ctx = int(c.ctx_lens.max().item())
    ws = torch.empty(max(kv.paged_multi_token_attention_workspace_bytes(pool, c.batch, c.n_h, 4, max_ctx), 256),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty(c.q.shape, dtype=torch.float32, device=DEV)
    kv.kv_decode_step(pool, c.k_new, c.v_new, c.q, out, c.tables, c.seq_lens, c.scale, max_ctx, ws)
    K, V = wl.to_host_bits(c.K), wl.to_host_bits(c.V)
    tab, sl = c.tables.cpu().numpy(), c.seq_lens.cpu().numpy()
    kn, vn = wl.to_host_bits(c.k_new), wl.to_host_bits(c.v_new)
    for t in range(4):  # the oracle appends one token per call
        orc.append(K, V, np.ascontiguousarray(kn[:, t]), np.ascontiguousarray(vn[:, t]), tab, sl + t)
    assert np.array_equal(wl.to_host_bits(pool.K), K) and np.array_equal(wl.to_host_bits(pool.V), V)
    want = orc.attention_multi(K, V, wl.to_host_bits(c.q), tab, c.ctx_lens.cpu().numpy(), c.scale)
    got = out.cpu().numpy()
    assert np.abs(got - want).max() <= TOL
