"""Parity of the selective-recompute selection kernels with the oracle (GPU).

kv_token_deviation is fp64 on both sides; only the summation order differs,
so the test bound is 1e-12 relative. kv_topk_select is compared index for
index with the oracle's top-k on the very same fp64 values (an integer
result decided in the same precision on both sides). The end-to-end selection
(deviation then top-k) must match the oracle's except for rows whose oracle
deviation lies within rounding distance of the k-th largest.
"""
import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REL = 1e-12

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


def new_pool(c):
    p = kv.KVPool(c.num_blocks, c.n_kv, c.d, c.dtype, device=DEV)
    p.K.copy_(c.K)
    p.V.copy_(c.V)
    return p


def oracle_dev(c):
    return orc.deviation(wl.to_host_bits(c.K), wl.to_host_bits(c.V), wl.to_host_bits(c.tables),
                         c.row_seq.cpu().numpy(), c.row_pos.cpu().numpy(), wl.to_host_bits(c.k_re),
                         wl.to_host_bits(c.v_re))


def gpu_dev(pool, c):
    return kv.kv_token_deviation(pool, c.tables, c.row_seq, c.row_pos, c.k_re, c.v_re)


def assert_dev_close(got, want):
    got = np.asarray(got)
    assert got.shape == want.shape
    err = np.abs(got - want) / np.maximum(want, 1.0)
    assert err.max(initial=0.0) <= REL, f"max rel err {err.max()}"
    assert np.array_equal(got == 0.0, want == 0.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n_kv,d", [(1, 64), (3, 64), (2, 128), (8, 128)])
@pytest.mark.parametrize("rows_per_seq", [None, 37])
def test_deviation_parity(dtype, n_kv, d, rows_per_seq):
    print(f"deviation dtype={dtype} n_kv={n_kv} d={d} rows={rows_per_seq}", flush=True)
    c = wl.make_blend_case(11, 3, 181, n_kv, d, dtype, 0.1, rows_per_seq, DEV)
    pool = new_pool(c)
    got = gpu_dev(pool, c).cpu().numpy()
    torch.cuda.synchronize()
    assert_dev_close(got, oracle_dev(c))


def test_deviation_invalid_rows_get_minus_inf():
    c = wl.make_blend_case(12, 2, 64, 2, 64, "bf16", 0.0, None, DEV)
    pool = new_pool(c)
    rs, rp = c.row_seq.clone(), c.row_pos.clone()
    tables = c.tables.clone()
    rs[3] = 2            # no such sequence
    rs[5] = -1
    rp[7] = 64 * 16      # past the table
    rp[9] = -1
    tables[1, 2] = -1    # sequence 1, positions 32..47: unmapped block
    tables[1, 3] = c.num_blocks
    out = kv.kv_token_deviation(pool, tables, rs, rp, c.k_re, c.v_re).cpu().numpy()
    bad = np.zeros(c.n_rows, bool)
    bad[[3, 5, 7, 9]] = True
    seq, pos = c.row_seq.cpu().numpy(), c.row_pos.cpu().numpy()
    bad |= (seq == 1) & (pos >= 32) & (pos < 64)
    assert np.all(out[bad] == -np.inf)
    want = oracle_dev(c)
    assert_dev_close(out[~bad], want[~bad])


def test_deviation_empty_and_zero_rows():
    c = wl.make_blend_case(13, 2, 40, 2, 64, "bf16", 1.0, None, DEV)   # every row unchanged
    pool = new_pool(c)
    assert np.all(gpu_dev(pool, c).cpu().numpy() == 0.0)
    e = torch.zeros(0, dtype=torch.int32, device=DEV)
    out = kv.kv_token_deviation(pool, c.tables, e, e, c.k_re[:0], c.v_re[:0])
    assert out.numel() == 0


def oracle_topk_segments(vals, offs, ks):
    out = []
    for s in range(len(ks)):
        seg = vals[offs[s]:offs[s + 1]]
        out.append(orc.topk(seg, max(int(ks[s]), 0)) if len(seg) else np.zeros(0, np.int32))
    return out


def run_topk(vals, offs, ks):
    v = torch.tensor(vals, dtype=torch.float64, device=DEV)
    o = torch.tensor(offs, dtype=torch.int32, device=DEV)
    k = torch.tensor(ks, dtype=torch.int32, device=DEV)
    sel = kv.kv_topk_select(v, o, k).cpu().numpy()
    return sel


def check_topk(vals, offs, ks):
    sel = run_topk(vals, offs, ks)
    want = oracle_topk_segments(vals, offs, ks)
    for s in range(len(ks)):
        n = offs[s + 1] - offs[s]
        m = min(max(int(ks[s]), 0), n)
        got = sel[offs[s]:offs[s] + m]
        assert np.array_equal(got, want[s]), f"segment {s} (n={n}, k={ks[s]})"
        assert np.all(sel[offs[s] + m:offs[s + 1]] == -1), f"segment {s} wrote past its count"


@pytest.mark.parametrize("kind", ["normal", "ties", "constant", "signed", "special"])
def test_topk_parity(kind):
    rng = np.random.default_rng(["normal", "ties", "constant", "signed", "special"].index(kind) + 80)
    lens = [0, 1, 2, 5, 63, 64, 65, 1000, 1023, 1024, 1025, 4097, 70000]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    total = int(offs[-1])
    if kind == "normal":
        vals = rng.standard_normal(total)
    elif kind == "ties":
        vals = rng.integers(0, 7, total).astype(np.float64)
    elif kind == "constant":
        vals = np.full(total, 2.5)
    elif kind == "signed":
        vals = rng.integers(-3, 4, total).astype(np.float64)
        vals[vals == 0] = np.where(rng.random(int((vals == 0).sum())) < 0.5, -0.0, 0.0)
    else:
        vals = rng.standard_normal(total) * 1e300
        vals[rng.random(total) < 0.05] = np.inf
        vals[rng.random(total) < 0.05] = -np.inf
        vals[rng.random(total) < 0.05] = 5e-324   # smallest subnormal
    for kfun in (lambda n: 1, lambda n: (n * 15 + 99) // 100, lambda n: n - 1, lambda n: n, lambda n: n + 3,
                 lambda n: 0, lambda n: -2, lambda n: n // 2):
        ks = [kfun(n) for n in lens]
        print(f"topk kind={kind} ks={ks[-3:]}", flush=True)
        check_topk(vals, offs, ks)


def test_topk_no_segments_and_empty():
    v = torch.zeros(4, dtype=torch.float64, device=DEV)
    o = torch.zeros(1, dtype=torch.int32, device=DEV)
    k = torch.zeros(0, dtype=torch.int32, device=DEV)
    assert np.all(kv.kv_topk_select(v, o, k).cpu().numpy() == -1)
    # segments of length 0 (a non-null buffer: the host never reads the offsets)
    sel = kv.kv_topk_select(v, torch.zeros(3, dtype=torch.int32, device=DEV),
                            torch.tensor([3, 0], dtype=torch.int32, device=DEV)).cpu().numpy()
    assert np.all(sel == -1)
    # a negative-length segment is skipped
    sel = kv.kv_topk_select(v, torch.tensor([3, 1, 4], dtype=torch.int32, device=DEV),
                            torch.tensor([2, 2], dtype=torch.int32, device=DEV)).cpu().numpy()
    assert list(sel) == [-1, 0, 1, -1]     # segment 1 = values[1:4], all equal: rows 0, 1


def test_topk_full_length_segment():
    """One long segment (a 128K-token context) at the 15 % floor."""
    rng = np.random.default_rng(90)
    n = 131072
    vals = rng.random(n) * 4096.0
    vals[rng.random(n) < 0.02] = 0.0
    check_topk(vals, [0, n], [orc.recompute_count(0.15, n)])


def select_and_check(c, ratio):
    """Deviation then top-k per request on the GPU, against the oracle's."""
    pool = new_pool(c)
    offs = c.seg_offsets.cpu().numpy()
    lens = np.diff(offs)
    ks = [kv.kv_recompute_count(ratio, int(n)) for n in lens]
    dev = gpu_dev(pool, c)
    sel = kv.kv_topk_select(dev, c.seg_offsets, torch.tensor(ks, dtype=torch.int32, device=DEV)).cpu().numpy()
    want_dev = oracle_dev(c)
    for s in range(c.batch):
        d = want_dev[offs[s]:offs[s + 1]]
        want = orc.topk(d, ks[s])
        got = sel[offs[s]:offs[s] + ks[s]]
        if np.array_equal(got, want):
            continue
        # only rows within rounding distance of the threshold may differ
        thr = np.sort(d)[::-1][ks[s] - 1]
        diff = np.setxor1d(got, want)
        assert len(got) == ks[s] and len(np.unique(got)) == ks[s]
        assert np.all(np.abs(d[diff] - thr) <= REL * max(thr, 1.0)), f"request {s}: {diff}"
    return dev.cpu().numpy(), want_dev


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_select_end_to_end(dtype):
    c = wl.make_blend_case(14, 5, 777, 8, 128, dtype, 0.05, None, DEV)
    select_and_check(c, 0.15)
    select_and_check(c, 0.5)


def test_select_narrowed_candidates():
    """A narrowed candidate set: rows are a seeded subset of each request's
    tokens; the selection indexes rows, mapped back through row_pos."""
    c = wl.make_blend_case(15, 4, 2048, 8, 128, "bf16", 0.05, 300, DEV)
    dev, _ = select_and_check(c, 0.25)
    assert np.all(dev >= 0.0)


def test_select_full_size_workload():
    c = wl.blend_workload("blend_select", DEV)
    print(f"blend_select rows={c.n_rows}", flush=True)
    got, want = select_and_check(c, wl.BLEND_WORKLOADS["blend_select"]["ratio"])
    assert_dev_close(got, want)
