"""Parity of the HIP path with the oracle (GPU).

Every test here calls the library through its C ABI (ctypes binding) on
cuda:0 and compares with the oracle on host copies of the very same inputs:
bit-exact for append, INT4 coding and RoPE; max |error| <= 2e-3 for attention
(fp32 outputs vs fp64 oracle). Unused pool slots hold NaN so that a stray
read shows up as NaN in the output.
"""
import copy

import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

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


DEV = "cuda:0"


def bits(t):
    return wl.to_host_bits(t)


def ibits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


def new_pool(c, dtype=None):
    p = kv.KVPool(c.num_blocks, c.n_kv, c.d, dtype or c.dtype, device=DEV)
    p.K.copy_(c.K)
    p.V.copy_(c.V)
    return p


def gpu_attention(pool, c, kernel=0, split_blocks=0, window=0, seq_slots=None, ctx=None, max_ctx=None, schedule=0):
    ctx = c.ctx_lens if ctx is None else ctx
    if max_ctx is None:
        max_ctx = int(ctx.max().item()) if ctx.numel() else 0
    opts = kv.attn_opts(split_blocks=split_blocks, kernel=kernel, window=window, schedule=schedule)
    nbytes = kv.paged_decode_attention_workspace_bytes(pool, c.batch, c.n_h, max_ctx, opts)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV)
    out = torch.full((c.batch, c.n_h, c.d), float("nan"), dtype=torch.float32, device=DEV)
    kv.paged_decode_attention(pool, c.q, out, c.tables, ctx, c.scale, max_ctx, ws, seq_slots, opts)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def oracle_step(c):
    """Host pool images after the oracle's append, and the oracle attention."""
    K, V = bits(c.K), bits(c.V)
    tab = c.tables.cpu().numpy()
    if c.append:
        orc.append(K, V, bits(c.k_new), bits(c.v_new), tab, c.seq_lens.cpu().numpy())
    return K, V


def max_err(a, b):
    return float(np.max(np.abs(a - b))) if a.size else 0.0


# ---------------------------------------------------------------------------
# append
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_append_bit_exact(dtype, d):
    c = wl.make_case(101, 6, [0, 15, 16, 17, 37, 50], 8, 2, d, dtype, num_blocks=24, device=DEV)
    pool = new_pool(c)
    kv.kv_append(pool, c.k_new, c.v_new, c.tables, c.seq_lens)
    torch.cuda.synchronize()
    K, V = oracle_step(c)
    assert np.array_equal(ibits(bits(pool.K)), ibits(K))
    assert np.array_equal(ibits(bits(pool.V)), ibits(V))


def test_append_skips_rows_with_bad_metadata():
    c = wl.make_case(102, 3, [5, 20, 33], 4, 2, 64, "bf16", num_blocks=8, device=DEV)
    pool = new_pool(c)
    lens = c.seq_lens.clone()
    lens[1] = -3                          # invalid length: that row is skipped
    tab = c.tables.clone()
    tab[2, 33 // 16] = 10_000             # block id out of range: skipped
    kv.kv_append(pool, c.k_new, c.v_new, tab, lens)
    torch.cuda.synchronize()
    K, V = bits(c.K), bits(c.V)
    orc.append(K[:], V[:], bits(c.k_new)[:1], bits(c.v_new)[:1], c.tables.cpu().numpy()[:1],
               c.seq_lens.cpu().numpy()[:1])
    assert np.array_equal(bits(pool.K), K) and np.array_equal(bits(pool.V), V)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def test_tiny_workload():
    """Both sequences of the tiny fp32 workload, append then attend."""
    c = wl.workload("tiny", device=DEV)
    pool = new_pool(c)
    kv.kv_append(pool, c.k_new, c.v_new, c.tables, c.seq_lens)
    out = gpu_attention(pool, c)
    K, V = oracle_step(c)
    assert np.array_equal(ibits(bits(pool.K)), ibits(K))
    ref = orc.attention(K, V, bits(c.q), c.tables.cpu().numpy(), c.ctx_lens.cpu().numpy(), c.scale)
    assert max_err(out, ref) <= TOL


SHAPES = [
    # (lens, n_h, n_kv, d, dtype)
    ([1, 2, 15, 16, 17, 33], 4, 2, 64, "f32"),
    ([1, 16, 31, 300, 17], 8, 8, 128, "bf16"),
    ([5, 64, 129, 250], 8, 1, 128, "bf16"),
    ([3, 47, 96, 200], 32, 8, 128, "bf16"),
    ([7, 48, 255, 256], 64, 8, 128, "bf16"),
    ([12, 90, 161], 16, 1, 64, "bf16"),
    ([40, 1, 77], 6, 2, 128, "bf16"),
    ([40, 1, 77], 6, 2, 64, "f32"),
    ([23, 260], 16, 4, 128, "f32"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[4]}-g{s[1]//s[2]}-d{s[3]}" for s in SHAPES])
@pytest.mark.parametrize("kernel", [1, 2])
@pytest.mark.parametrize("split", [0, 1, 3])
def test_attention_parity(shape, kernel, split):
    lens, n_h, n_kv, d, dtype = shape
    if kernel == 2 and dtype != "bf16":
        pytest.skip("MFMA path is bf16 only")
    c = wl.make_case(200 + len(lens) + n_h, len(lens), lens, n_h, n_kv, d, dtype, device=DEV)
    pool = new_pool(c)
    kv.kv_append(pool, c.k_new, c.v_new, c.tables, c.seq_lens)
    out = gpu_attention(pool, c, kernel=kernel, split_blocks=split)
    K, V = oracle_step(c)
    ref = orc.attention(K, V, bits(c.q), c.tables.cpu().numpy(), c.ctx_lens.cpu().numpy(), c.scale)
    assert np.all(np.isfinite(out))
    assert max_err(out, ref) <= TOL


def add_score_ramp(c, amp):
    """Adds to every attended key row a multiple of its query group's mean
    direction that grows with the token position: the scores then rise by
    about 0.7 * amp log2 units over each sequence, so the running maximum keeps
    moving, in steps both above and below the MFMA paths' rescaling slack."""
    K = c.K.float().cpu()
    q = c.q.float().cpu()
    g = c.n_h // c.n_kv
    u = q.view(c.batch, c.n_kv, g, c.d).mean(2)
    u = u / u.norm(dim=-1, keepdim=True).clamp_min(1e-6)
    tab = c.tables.cpu()
    for b in range(c.batch):
        n = int(c.ctx_lens[b])
        for j in range(n):
            K[int(tab[b, j // 16]), :, j % 16, :] += amp * (j / max(n - 1, 1)) * u[b]
    c.K.copy_(K.to(c.K.dtype))


@pytest.mark.parametrize("n_h", [32, 64])
@pytest.mark.parametrize("amp", [12.0, 60.0])
@pytest.mark.parametrize("dtype", ["bf16", "int4"])
@pytest.mark.parametrize("split", [0, 3])
def test_rising_scores(n_h, amp, dtype, split):
    """Scores that climb along the sequence (the running maximum moves on most
    tiles): the MFMA paths against the oracle, both schedules."""
    lens = [300, 1000, 17, 2000, 40]
    c = wl.make_case(260 + n_h + int(amp), len(lens), lens, n_h, 8, 128, "bf16", append=False, device=DEV)
    add_score_ramp(c, amp)
    tab, ctx = c.tables.cpu().numpy(), c.ctx_lens.cpu().numpy()
    if dtype == "bf16":
        pool = new_pool(c)
        out = gpu_attention(pool, c, kernel=2, split_blocks=split)
        Kr, Vr = bits(c.K), bits(c.V)
    else:
        slots = torch.arange(len(lens), dtype=torch.int32, device=DEV)
        src, dst, img = int4_pools(c, len(lens))
        kv.kv_quantize_int4(dst, src, c.tables, c.ctx_lens, slots)
        orc.q4_quantize_pool(img, bits(c.K), bits(c.V), tab, ctx, slots.cpu().numpy())
        assert_img_equal(dst, img)
        out = gpu_attention(dst, c, kernel=2, split_blocks=split, seq_slots=slots)
        Kr, Vr = orc.q4_dequant(img, tab, ctx, slots.cpu().numpy())
    ref = orc.attention(Kr, Vr, bits(c.q), tab, ctx, c.scale)
    assert np.all(np.isfinite(out))
    assert max_err(out, ref) <= TOL


@pytest.mark.parametrize("g,q_len", [(8, 1), (4, 2), (2, 8)])
@pytest.mark.parametrize("window", [0, 30])
def test_many_units_merge(g, q_len, window):
    """300 sequences x 8 kv heads (2400 units of 8 or 16 query columns: the
    merge with one workgroup per unit), lengths 0-400 with empty sequences."""
    r = np.random.default_rng(70 + g + q_len)
    lens = [int(x) for x in r.integers(q_len, 400, 300)]
    lens[5] = lens[17] = 0
    c = wl.make_case(980 + g, len(lens), lens, 8 * g, 8, 128, "bf16", append=False, device=DEV)
    pool = new_pool(c)
    gq = torch.Generator(device=DEV).manual_seed(g)
    q = torch.randn((c.batch, q_len, 8 * g, 128), generator=gq, device=DEV).to(torch.bfloat16)
    out = gpu_multi(pool, c, q, window=window, schedule=2)
    ref = orc.attention_multi(bits(c.K), bits(c.V), bits(q), c.tables.cpu().numpy(), c.ctx_lens.cpu().numpy(),
                              c.scale, window=window)
    assert np.all(np.isfinite(out))
    assert max_err(out, ref) <= TOL


@pytest.mark.parametrize("schedule,split", [(0, 0), (1, 70000), (1, 300)])
def test_million_token_context(schedule, split):
    """A 1,000,000-token sequence beside a short one (bf16, MFMA): the
    balanced schedule, one split over the whole sequence (62,500 blocks, far
    more block ids than a workgroup stages at once) and 300-block splits."""
    lens = [1_000_000, 5000]
    c = wl.make_case(901, len(lens), lens, 8, 1, 64, "bf16", append=False, device=DEV)
    pool = new_pool(c)
    out = gpu_attention(pool, c, kernel=2, split_blocks=split, schedule=schedule)
    ref = orc.attention(bits(c.K), bits(c.V), bits(c.q), c.tables.cpu().numpy(), c.ctx_lens.cpu().numpy(), c.scale)
    assert np.all(np.isfinite(out))
    assert max_err(out, ref) <= TOL


def test_int4_long_context():
    """INT4 over 300,000 tokens in one split (18,750 blocks) and balanced."""
    lens = [300_000, 33]
    c = wl.make_case(902, len(lens), lens, 8, 1, 128, "bf16", append=False, device=DEV, outliers=4)
    slots = torch.arange(len(lens), dtype=torch.int32, device=DEV)
    src, dst, img = int4_pools(c, len(lens))
    kv.kv_quantize_int4(dst, src, c.tables, c.ctx_lens, slots)
    tab, ctx, sl = c.tables.cpu().numpy(), c.ctx_lens.cpu().numpy(), slots.cpu().numpy()
    orc.q4_quantize_pool(img, bits(c.K), bits(c.V), tab, ctx, sl)
    assert_img_equal(dst, img)
    Kd, Vd = orc.q4_dequant(img, tab, ctx, sl)
    ref = orc.attention(Kd, Vd, bits(c.q), tab, ctx, c.scale)
    for schedule, split in [(0, 0), (1, 20000)]:
        out = gpu_attention(dst, c, kernel=2, split_blocks=split, schedule=schedule, seq_slots=slots)
        assert np.all(np.isfinite(out))
        assert max_err(out, ref) <= TOL


@pytest.mark.parametrize("kernel,split", [(1, 2), (2, 2), (2, 0)])
def test_permutation_and_repeat_are_bit_identical(kernel, split):
    c = wl.make_case(300, 4, [70, 15, 128, 99], 16, 4, 128, "bf16", num_blocks=40, append=False, device=DEV)
    pool = new_pool(c)
    a = gpu_attention(pool, c, kernel=kernel, split_blocks=split)
    b = gpu_attention(pool, c, kernel=kernel, split_blocks=split)
    assert np.all(np.isfinite(a)) and np.array_equal(a, b)
    perm = torch.randperm(c.num_blocks, generator=torch.Generator().manual_seed(5)).to(DEV)
    pool2 = kv.KVPool(c.num_blocks, c.n_kv, c.d, "bf16", device=DEV)
    pool2.K[perm.long()] = c.K
    pool2.V[perm.long()] = c.V
    tab2 = torch.where(c.tables >= 0, perm[c.tables.clamp(min=0).long()].to(torch.int32), c.tables)
    c2 = wl.Case(**{**c.__dict__, "tables": tab2.contiguous()})
    moved = gpu_attention(pool2, c2, kernel=kernel, split_blocks=split)
    assert np.array_equal(a, moved)


@pytest.mark.parametrize("window", [1, 5, 16, 17, 100, 1000])
@pytest.mark.parametrize("kernel,split", [(1, 2), (2, 2), (2, 0)])
def test_window(window, kernel, split):
    c = wl.make_case(400, 5, [0, 9, 40, 130, 333], 8, 2, 128, "bf16", device=DEV)
    pool = new_pool(c)
    kv.kv_append(pool, c.k_new, c.v_new, c.tables, c.seq_lens)
    out = gpu_attention(pool, c, kernel=kernel, window=window, split_blocks=split)
    K, V = oracle_step(c)
    ref = orc.attention(K, V, bits(c.q), c.tables.cpu().numpy(), c.ctx_lens.cpu().numpy(), c.scale,
                        window=window)
    assert max_err(out, ref) <= TOL


@pytest.mark.parametrize("kernel,split", [(1, 1), (2, 1), (2, 0)])
def test_empty_context_and_bad_metadata(kernel, split):
    c = wl.make_case(500, 4, [0, 20, 40, 60], 8, 2, 128, "bf16", append=False, device=DEV)
    pool = new_pool(c)
    tab = c.tables.clone()
    tab[0, 0] = 0                           # seq 0 attends nothing: table entry unused
    tab[2, 1] = 99_999                      # seq 2 names a block outside the pool
    ctx = c.ctx_lens.clone()
    ctx[3] = 10_000                         # seq 3 claims more tokens than its table holds
    c2 = wl.Case(**{**c.__dict__, "tables": tab.contiguous()})
    out = gpu_attention(pool, c2, kernel=kernel, split_blocks=split, ctx=ctx, max_ctx=60)
    assert np.all(out[0] == 0.0)
    assert np.all(np.isnan(out[2])) and np.all(np.isnan(out[3]))
    ref = orc.attention(bits(c.K), bits(c.V), bits(c.q), c.tables.cpu().numpy(), c.ctx_lens.cpu().numpy(), c.scale)
    assert max_err(out[1], ref[1]) <= TOL


def test_error_codes_on_device_call():
    c = wl.make_case(600, 2, [10, 20], 8, 2, 128, "bf16", device=DEV)
    pool = new_pool(c)
    out = torch.empty((2, 8, 128), dtype=torch.float32, device=DEV)
    with pytest.raises(kv.KVError) as e:
        kv.paged_decode_attention(pool, c.q, out, c.tables, c.ctx_lens, c.scale, 21, None, opts=kv.attn_opts(split_blocks=1))
    assert e.value.status == kv.KV_ERR_WORKSPACE
    with pytest.raises(kv.KVError) as e:
        kv.paged_decode_attention(pool, c.q, out, c.tables, c.ctx_lens, c.scale, 400, None)
    assert e.value.status == kv.KV_ERR_INVALID_ARG
    f32q = c.q.float()
    with pytest.raises(ValueError):
        kv.paged_decode_attention(pool, f32q, out, c.tables, c.ctx_lens, c.scale, 21)


@pytest.mark.parametrize("window", [0, 300])
def test_schedules_agree(window):
    """Balanced and fixed-split schedules cut the context differently; both
    stay within the bound of the oracle."""
    lens = [int(x) for x in torch.randint(0, 900, (37,), generator=torch.Generator().manual_seed(3))]
    c = wl.make_case(901, 37, lens, 32, 8, 128, "bf16", device=DEV)
    pool = new_pool(c)
    kv.kv_append(pool, c.k_new, c.v_new, c.tables, c.seq_lens)
    K, V = oracle_step(c)
    ref = orc.attention(K, V, bits(c.q), c.tables.cpu().numpy(), c.ctx_lens.cpu().numpy(), c.scale, window=window)
    for split in (0, 1, 5, 64):
        out = gpu_attention(pool, c, kernel=2, split_blocks=split, window=window)
        assert max_err(out, ref) <= TOL, split


@pytest.mark.parametrize("lens,n_h,n_kv,window", [([40000], 8, 1, 0), ([0, 17, 30000], 4, 1, 0),
                                                   ([25000, 9], 16, 2, 20000)])
def test_balanced_merge_many_partials(lens, n_h, n_kv, window):
    """Few long sequences over the whole persistent grid: one (sequence, kv
    head) pair is cut across hundreds of workgroups, so the merge combines its
    partials in several chunks of 64."""
    c = wl.make_case(907, len(lens), lens, n_h, n_kv, 128, "bf16", device=DEV)
    pool = new_pool(c)
    kv.kv_append(pool, c.k_new, c.v_new, c.tables, c.seq_lens)
    K, V = oracle_step(c)
    ref = orc.attention(K, V, bits(c.q), c.tables.cpu().numpy(), c.ctx_lens.cpu().numpy(), c.scale, window=window)
    out = gpu_attention(pool, c, kernel=2, window=window, schedule=2)
    assert max_err(out, ref) <= TOL


# The full-size workloads, every row on the path bench.py times, are in
# test_gpu_full_size.py.


# ---------------------------------------------------------------------------
# shared-prefix decode attention
# ---------------------------------------------------------------------------

def shared_case(seed, lens, n_h, n_kv, d, groups):
    """A case whose group members' tables name their first member's physical
    blocks for the group's prefix (the members' own first blocks go unused)."""
    c = wl.make_case(seed, len(lens), lens, n_h, n_kv, d, "bf16", append=False, device=DEV)
    t = c.tables.clone()
    for (a, b), P in zip(zip(groups[0][:-1], groups[0][1:]), groups[1]):
        for m in range(a + 1, b):
            t[m, :P] = t[a, :P]
    c.tables = t
    return c


def gpu_shared(pool, c, group_start, prefix_blocks, split_blocks=0, schedule=0):
    g = kv.prefix_groups(group_start, prefix_blocks)
    opts = kv.attn_opts(split_blocks=split_blocks, schedule=schedule)
    max_ctx = int(c.ctx_lens.max().item())
    nbytes = kv.paged_decode_attention_shared_workspace_bytes(pool, c.batch, c.n_h, max_ctx, g, opts)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV)
    out = torch.full((c.batch, c.n_h, c.d), float("nan"), dtype=torch.float32, device=DEV)
    kv.paged_decode_attention_shared(pool, c.q, out, c.tables, c.ctx_lens, c.scale, max_ctx, g, ws, opts)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


SHARED_CASES = [
    # lens, n_h, n_kv, d, (group_start, prefix_blocks)
    ([300, 700, 520, 1000, 64], 8, 2, 128, ([0, 3, 4], [10, 5])),      # a group of 3, a group of 1, one outside
    ([260, 250, 400, 210, 390, 300, 90], 8, 2, 128, ([0, 6], [12])),     # 6 members x 4 heads: 2 column tiles
    ([400, 320, 330, 1000], 4, 4, 128, ([0, 4], [20])),                 # MHA; a member with no own block
    ([180, 90, 400, 64, 100], 4, 1, 64, ([0, 0, 2, 4], [3, 4, 2])),    # MQA, d 64, an empty group
    ([17, 33, 48, 1], 2, 2, 128, ([1, 3], [1])),                        # ragged tails, tiny prefix
]


@pytest.mark.parametrize("case", range(len(SHARED_CASES)))
@pytest.mark.parametrize("schedule,split", [(0, 0), (2, 0), (1, 0), (1, 1), (1, 5)])
def test_shared_prefix_parity(case, schedule, split):
    """Balanced (auto and explicit) and item schedules of the shared-prefix call."""
    lens, n_h, n_kv, d, groups = SHARED_CASES[case]
    c = shared_case(60 + case, lens, n_h, n_kv, d, groups)
    pool = new_pool(c)
    out = gpu_shared(pool, c, groups[0], groups[1], split_blocks=split, schedule=schedule)
    ref = orc.attention(bits(c.K), bits(c.V), bits(c.q), c.tables.cpu().numpy(), c.ctx_lens.cpu().numpy(), c.scale)
    assert max_err(out, ref) <= TOL


@pytest.mark.parametrize("schedule,split", [(1, 1000), (0, 0)])
def test_shared_prefix_items_longer_than_the_id_window(schedule, split):
    """Prefix and suffix segments of 400-850 blocks (items of 1000 blocks, or
    the balanced shares): the kernels run them in pieces of 256 blocks."""
    lens = [20000, 16000, 9000]
    groups = ([0, 3], [400])
    c = shared_case(75, lens, 8, 2, 128, groups)
    pool = new_pool(c)
    out = gpu_shared(pool, c, groups[0], groups[1], split_blocks=split, schedule=schedule)
    ref = orc.attention(bits(c.K), bits(c.V), bits(c.q), c.tables.cpu().numpy(), c.ctx_lens.cpu().numpy(), c.scale)
    assert max_err(out, ref) <= TOL


@pytest.mark.parametrize("schedule", [0, 1])
def test_shared_prefix_member_shorter_than_prefix_is_nan(schedule):
    c = shared_case(71, [300, 100, 250], 4, 2, 128, ([0, 2], [10]))   # member 1 has 100 < 160 prefix tokens
    pool = new_pool(c)
    out = gpu_shared(pool, c, [0, 2], [10], schedule=schedule)
    assert np.isnan(out[1]).all()
    keep = [0, 2]
    ref = orc.attention(bits(c.K), bits(c.V), bits(c.q)[keep], c.tables.cpu().numpy()[keep],
                        c.ctx_lens.cpu().numpy()[keep], c.scale)
    assert max_err(out[keep], ref) <= TOL


def test_shared_prefix_long_workload_matches_plain_call():
    """The long shared-prefix workload (8 x 32768 tokens, 16384 shared, chunk
    re-rotated) through the shared entry point and through the plain call:
    every row of the two agrees (each is checked against the oracle on every
    row in test_gpu_full_size.py and here at small sizes)."""
    c = wl.workload("long_shared", device=DEV)
    pool = new_pool(c)
    kv.rope_rerotate(pool, c.chunk_blocks, 0, c.chunk_tokens, c.delta, c.rope_base, 0)
    out = gpu_shared(pool, c, [0, c.batch], [1024])
    plain = gpu_attention(pool, c)
    assert np.all(np.isfinite(out))
    assert max_err(out, plain) <= TOL


# ---------------------------------------------------------------------------
# RoPE re-rotation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("style", [0, 1])
@pytest.mark.parametrize("first_slot,num_tokens,delta", [(0, 48, 1), (3, 40, 9876), (5, 1, -77), (0, 64, 16384)])
def test_rope_bit_exact(dtype, style, first_slot, num_tokens, delta):
    c = wl.make_case(700, 1, [64], 4, 4, 128, dtype, append=False, poison=False, device=DEV)
    pool = new_pool(c)
    kv.rope_rerotate(pool, c.tables[0], first_slot, num_tokens, delta, 10000.0, style)
    torch.cuda.synchronize()
    K = bits(c.K)
    orc.rope_rerotate(K, c.tables.cpu().numpy()[0], first_slot, num_tokens, delta, 10000.0, style)
    assert np.array_equal(ibits(bits(pool.K)), ibits(K))
    assert np.array_equal(ibits(bits(pool.V)), ibits(bits(c.V)))


# ---------------------------------------------------------------------------
# INT4
# ---------------------------------------------------------------------------

def int4_pools(c, max_seqs):
    src = new_pool(c, "bf16")
    dst = kv.KVPool(c.num_blocks, c.n_kv, c.d, "int4", max_seqs=max_seqs, device=DEV)
    dst.blob.fill_(0x5A)
    img = orc.Q4Image(c.num_blocks, c.n_kv, c.d, max_seqs)
    for a in img.arrays():
        a.view(np.uint8)[...] = 0x5A
    return src, dst, img


def assert_img_equal(dst, img):
    pairs = [(dst.KQ, img.kq), (dst.KS, img.ks), (dst.KM, img.km), (dst.VQ, img.vq), (dst.VS, img.vs),
             (dst.VM, img.vm), (dst.KTAIL, img.kt)]
    for t, a in pairs:
        h = t.detach().cpu().contiguous()
        h = h.view(torch.int16).numpy().view(np.uint16) if h.element_size() == 2 else h.numpy()
        assert np.array_equal(h, a)


def int4_case(seed, lens, n_h=8, n_kv=2, d=128, outliers=4):
    return wl.make_case(seed, len(lens), lens, n_h, n_kv, d, "bf16", device=DEV, outliers=outliers)


def tie_values(shape_rows, n, which):
    """Rows of n values whose INT4 quotients (x - min) / s are exact
    half-integers: row i uses (min, s) = PAIRS[i % 3]; element 0 is the min,
    element 1 the max (min + 15 s), element j the min + ((j + i) % 15 + 0.5) s.
    All values are exact in bf16 and fp16, and s = (max - min) / 15 exactly."""
    pairs = [(0.0, 0.25), (-1.0, 0.125), (2.0, 0.5)]
    out = np.empty(shape_rows + (n,), dtype=np.float32)
    idx = np.arange(n)
    flat = out.reshape(-1, n)
    for i in range(flat.shape[0]):
        m, sc = pairs[(i + which) % 3]
        v = m + (((idx + i) % 15) + 0.5) * sc
        v[0], v[1] = m, m + 15 * sc
        flat[i] = v
    return out


@pytest.mark.parametrize("fused", [False, True])
def test_int4_exact_ties_round_half_away(fused):
    """Groups whose quotients are exact half-integers (the rounding rule's
    hard case): bulk coding, then an append that completes a block, bit-exact
    against the oracle; with fused=True the append is the decode step's."""
    lens = [31, 20]
    c = int4_case(830, lens, n_h=4, n_kv=2, d=128, outliers=0)
    nb, nkv, d = c.num_blocks, c.n_kv, c.d
    # V: per token row over channels; K: per channel over a block's 16 tokens
    v = tie_values((nb, nkv, 16), d, 0)
    k = np.swapaxes(tie_values((nb, nkv, d), 16, 1), -1, -2).copy()
    c.V.copy_(torch.from_numpy(v).to(DEV, torch.bfloat16))
    c.K.copy_(torch.from_numpy(k).to(DEV, torch.bfloat16))
    # the new tokens continue the patterns at their slots
    knew = np.empty((2, nkv, d), dtype=np.float32)
    vnew = tie_values((2, nkv), d, 2)
    for b, L in enumerate(lens):
        t = L % 16
        knew[b] = k[0, :, t, :]
    c.k_new.copy_(torch.from_numpy(knew).to(DEV, torch.bfloat16))
    c.v_new.copy_(torch.from_numpy(vnew).to(DEV, torch.bfloat16))
    slots = torch.tensor([1, 0], dtype=torch.int32, device=DEV)
    src, dst, img = int4_pools(c, 2)
    kv.kv_quantize_int4(dst, src, c.tables, c.seq_lens, slots)
    tab, ln, sl = c.tables.cpu().numpy(), c.seq_lens.cpu().numpy(), slots.cpu().numpy()
    orc.q4_quantize_pool(img, bits(c.K), bits(c.V), tab, ln, sl)
    torch.cuda.synchronize()
    assert_img_equal(dst, img)
    if fused:
        max_ctx = int(c.ctx_lens.max().item())
        ws = torch.empty(max(kv.paged_decode_attention_workspace_bytes(dst, 2, c.n_h, max_ctx), 256),
                         dtype=torch.uint8, device=DEV)
        out = torch.empty((2, c.n_h, d), dtype=torch.float32, device=DEV)
        kv.kv_decode_step(dst, c.k_new, c.v_new, c.q, out, c.tables, c.seq_lens, c.scale, max_ctx, ws,
                          seq_slots=slots)
    else:
        kv.kv_append(dst, c.k_new, c.v_new, c.tables, c.seq_lens, slots)
    torch.cuda.synchronize()
    orc.q4_append(img, bits(c.k_new), bits(c.v_new), tab, ln, sl)
    assert_img_equal(dst, img)
    # the codes really are the half-away-from-zero roundings: V row i (token 0
    # of the first block of sequence 0, kv head 0) holds codes 0, 15 and
    # ((j + i) % 15) + 1 for its ties
    pid = int(tab[0, 0])
    i = pid * nkv * 16
    row = img.vq[pid, 0, 0]
    codes = np.stack([row & 15, row >> 4], axis=1).reshape(-1)
    want = np.array([0, 15] + [((j + i) % 15) + 1 for j in range(2, d)])
    assert np.array_equal(codes, want)


@pytest.mark.parametrize("d", [64, 128])
def test_int4_bulk_then_append_bit_exact(d):
    c = int4_case(800, [0, 14, 15, 16, 17, 31, 47, 100], d=d)
    slots = torch.tensor([7, 6, 5, 4, 3, 2, 1, 0], dtype=torch.int32, device=DEV)
    src, dst, img = int4_pools(c, 8)
    kv.kv_quantize_int4(dst, src, c.tables, c.seq_lens, slots)
    torch.cuda.synchronize()
    tab, lens, sl = c.tables.cpu().numpy(), c.seq_lens.cpu().numpy(), slots.cpu().numpy()
    orc.q4_quantize_pool(img, bits(c.K), bits(c.V), tab, lens, sl)
    assert_img_equal(dst, img)
    kv.kv_append(dst, c.k_new, c.v_new, c.tables, c.seq_lens, slots)
    torch.cuda.synchronize()
    orc.q4_append(img, bits(c.k_new), bits(c.v_new), tab, lens, sl)
    assert_img_equal(dst, img)
    # attention over the INT4 pool vs the oracle on the same dequantized values
    out = gpu_attention(dst, c, seq_slots=slots)
    Kd, Vd = orc.q4_dequant(img, tab, c.ctx_lens.cpu().numpy(), sl)
    ref = orc.attention(Kd, Vd, bits(c.q), tab, c.ctx_lens.cpu().numpy(), c.scale)
    assert max_err(out, ref) <= TOL


def test_int4_append_many_steps():
    """20 appends in a row cross block boundaries and complete blocks."""
    c = wl.make_case(801, 2, [3, 30], 4, 2, 128, "bf16", num_blocks=12, device=DEV, outliers=4, poison=False)
    tab = torch.tensor([[9, 1, 4, -1, -1, -1, -1, -1], [3, 0, 11, 6, -1, -1, -1, -1]], dtype=torch.int32)
    c.tables = tab.to(DEV)
    src, dst, img = int4_pools(c, 2)
    lens = torch.tensor([3, 30], dtype=torch.int32, device=DEV)
    kv.kv_quantize_int4(dst, src, c.tables, lens)
    orc.q4_quantize_pool(img, bits(c.K), bits(c.V), tab.numpy(), lens.cpu().numpy())
    g = torch.Generator(device=DEV).manual_seed(9)
    for step in range(20):
        kn = torch.randn((2, 2, 128), generator=g, device=DEV).to(torch.bfloat16)
        vn = torch.randn((2, 2, 128), generator=g, device=DEV).to(torch.bfloat16)
        kv.kv_append(dst, kn, vn, c.tables, lens)
        orc.q4_append(img, bits(kn), bits(vn), tab.numpy(), lens.cpu().numpy())
        lens += 1
    torch.cuda.synchronize()
    assert_img_equal(dst, img)


@pytest.mark.parametrize("kernel,split", [(1, 0), (2, 0), (2, 1), (2, 3)])
@pytest.mark.parametrize("window", [0, 40])
def test_int4_attention_kernels(kernel, split, window):
    """INT4 attention (VALU and MFMA, both schedules) against the oracle on
    the same dequantized values; lengths cover empty, partial and full blocks."""
    lens = [0, 1, 15, 16, 17, 31, 32, 33, 100, 255, 256, 400]
    c = int4_case(820, lens, n_h=32, n_kv=8, d=128)
    slots = torch.arange(len(lens) - 1, -1, -1, dtype=torch.int32, device=DEV)
    src, dst, img = int4_pools(c, len(lens))
    kv.kv_quantize_int4(dst, src, c.tables, c.seq_lens, slots)
    kv.kv_append(dst, c.k_new, c.v_new, c.tables, c.seq_lens, slots)
    tab, lens_np, sl = c.tables.cpu().numpy(), c.seq_lens.cpu().numpy(), slots.cpu().numpy()
    orc.q4_quantize_pool(img, bits(c.K), bits(c.V), tab, lens_np, sl)
    orc.q4_append(img, bits(c.k_new), bits(c.v_new), tab, lens_np, sl)
    out = gpu_attention(dst, c, kernel=kernel, split_blocks=split, window=window, seq_slots=slots)
    Kd, Vd = orc.q4_dequant(img, tab, c.ctx_lens.cpu().numpy(), sl)
    ref = orc.attention(Kd, Vd, bits(c.q), tab, c.ctx_lens.cpu().numpy(), c.scale, window=window)
    assert np.all(np.isfinite(out))
    assert max_err(out, ref) <= TOL


# ---------------------------------------------------------------------------
# block copies
# ---------------------------------------------------------------------------

def _regions_host(pool):
    if pool.dtype == "int4":
        ts = [pool.KQ, pool.KS, pool.KM, pool.VQ, pool.VS, pool.VM]
    else:
        ts = [pool.K, pool.V]
    out = []
    for t in ts:
        h = t.detach().cpu().contiguous()
        out.append(h.view(torch.uint8).numpy().reshape(h.shape[0], -1).copy())
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16", "int4"])
def test_block_copy_gather_scatter(dtype):
    nb = 40
    pool = kv.KVPool(nb, 4, 128, dtype, max_seqs=2 if dtype == "int4" else 0, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(77)
    pool.blob.copy_(torch.randint(0, 256, (pool.blob.numel(),), generator=g, device=DEV, dtype=torch.uint8))
    regs = _regions_host(pool)
    src = torch.tensor([3, 17, 38, 0, 22], dtype=torch.int32, device=DEV)
    dst = torch.tensor([5, 1, 9, 39, 30], dtype=torch.int32, device=DEV)
    kv.kv_copy_blocks(pool, src, dst)
    torch.cuda.synchronize()
    orc.copy_blocks(regs, src.cpu().numpy(), dst.cpu().numpy())
    assert all(np.array_equal(a, b) for a, b in zip(_regions_host(pool), regs))
    per = kv.kv_block_bytes(pool)
    blocks = torch.tensor([39, 2, 30, 11], dtype=torch.int32, device=DEV)
    for where in ("device", "pinned"):
        buf = (torch.zeros(4 * per, dtype=torch.uint8, device=DEV) if where == "device"
               else torch.zeros(4 * per, dtype=torch.uint8).pin_memory())
        kv.kv_gather_blocks(pool, blocks, buf)
        torch.cuda.synchronize()
        ref = orc.gather_blocks(regs, blocks.cpu().numpy())
        assert np.array_equal(buf.cpu().numpy(), ref), where
    # restore into other blocks from pinned host memory
    back = torch.tensor([12, 13, 14, 15], dtype=torch.int32, device=DEV)
    kv.kv_scatter_blocks(pool, back, buf)
    torch.cuda.synchronize()
    orc.scatter_blocks(regs, back.cpu().numpy(), ref)
    assert all(np.array_equal(a, b) for a, b in zip(_regions_host(pool), regs))


def test_block_copy_skips_out_of_range_ids():
    pool = kv.KVPool(8, 2, 64, "bf16", device=DEV)
    pool.blob.fill_(3)
    regs = _regions_host(pool)
    kv.kv_copy_blocks(pool, torch.tensor([1, 99, 2], dtype=torch.int32, device=DEV),
                      torch.tensor([-4, 5, 6], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    orc.copy_blocks(regs, [2], [6])
    assert all(np.array_equal(a, b) for a, b in zip(_regions_host(pool), regs))


# ---------------------------------------------------------------------------
# several query tokens per sequence (speculative verification / chunked prefill)
# ---------------------------------------------------------------------------

def gpu_multi(pool, c, q, kernel=0, split_blocks=0, window=0, seq_slots=None, schedule=0):
    max_ctx = int(c.ctx_lens.max().item())
    B, k, n_h, d = q.shape
    opts = kv.attn_opts(split_blocks=split_blocks, kernel=kernel, window=window, schedule=schedule)
    nbytes = kv.paged_multi_token_attention_workspace_bytes(pool, B, n_h, k, max_ctx, opts)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV)
    out = torch.full((B, k, n_h, d), float("nan"), dtype=torch.float32, device=DEV)
    kv.paged_multi_token_attention(pool, q, out, c.tables, c.ctx_lens, c.scale, max_ctx, ws, seq_slots, opts)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("n_h,n_kv,k", [(8, 2, 4), (32, 8, 4), (64, 8, 2), (8, 8, 16), (16, 2, 3), (64, 8, 5)])
@pytest.mark.parametrize("split,window", [(0, 0), (2, 0), (0, 37), (3, 37)])
def test_multi_token_parity(n_h, n_kv, k, split, window):
    lens = [0, 2, 16, 17, 40, 100, 300]            # cache length with the k new tokens included
    c = wl.make_case(950 + k, len(lens), lens, n_h, n_kv, 128, "bf16", append=False, device=DEV)
    pool = new_pool(c)
    g = torch.Generator(device=DEV).manual_seed(k)
    q = torch.randn((c.batch, k, n_h, 128), generator=g, device=DEV).to(torch.bfloat16)
    out = gpu_multi(pool, c, q, split_blocks=split, window=window)
    ref = orc.attention_multi(bits(c.K), bits(c.V), bits(q), c.tables.cpu().numpy(), c.ctx_lens.cpu().numpy(),
                              c.scale, window=window)
    assert np.all(np.isfinite(out))
    assert max_err(out, ref) <= TOL


def test_multi_token_one_token_is_decode():
    c = wl.make_case(960, 5, [7, 33, 64, 100, 250], 32, 8, 128, "bf16", append=False, device=DEV)
    pool = new_pool(c)
    a = gpu_attention(pool, c, kernel=2)
    b = gpu_multi(pool, c, c.q.view(c.batch, 1, c.n_h, c.d), kernel=2)
    assert np.array_equal(a, b[:, 0])


@pytest.mark.parametrize("split", [0, 2])
def test_multi_token_int4(split):
    k = 4
    lens = [3, 16, 21, 47, 200]
    c = int4_case(970, lens, n_h=32, n_kv=8, d=128)
    c.append = False
    c.ctx_lens = c.seq_lens.clone()
    src, dst, img = int4_pools(c, len(lens))
    kv.kv_quantize_int4(dst, src, c.tables, c.seq_lens)
    tab, lens_np = c.tables.cpu().numpy(), c.seq_lens.cpu().numpy()
    orc.q4_quantize_pool(img, bits(c.K), bits(c.V), tab, lens_np)
    g = torch.Generator(device=DEV).manual_seed(3)
    q = torch.randn((c.batch, k, c.n_h, 128), generator=g, device=DEV).to(torch.bfloat16)
    out = gpu_multi(dst, c, q, split_blocks=split)
    Kd, Vd = orc.q4_dequant(img, tab, lens_np)
    ref = orc.attention_multi(Kd, Vd, bits(q), tab, lens_np, c.scale)
    assert max_err(out, ref) <= TOL


@pytest.mark.parametrize("n_h,k", [(16, 2), (8, 3), (8, 4), (16, 1)])
@pytest.mark.parametrize("split,window", [(0, 0), (0, 37), (2, 0), (3, 37)])
def test_multi_token_int4_few_columns(n_h, k, split, window):
    """INT4 with at most four query columns per kv head (1-2 query heads per
    kv head times 1-4 query tokens: the one-score-per-lane softmax), causal
    among the new tokens and with a window, both schedules, lengths with
    partial blocks and shorter than the query count."""
    lens = [3, 16, 21, 47, 200, 333, 2]
    c = int4_case(975 + n_h + k, lens, n_h=n_h, n_kv=8, d=128)
    c.append = False
    c.ctx_lens = c.seq_lens.clone()
    src, dst, img = int4_pools(c, len(lens))
    kv.kv_quantize_int4(dst, src, c.tables, c.seq_lens)
    tab, lens_np = c.tables.cpu().numpy(), c.seq_lens.cpu().numpy()
    orc.q4_quantize_pool(img, bits(c.K), bits(c.V), tab, lens_np)
    g = torch.Generator(device=DEV).manual_seed(5 + k)
    q = torch.randn((c.batch, k, c.n_h, 128), generator=g, device=DEV).to(torch.bfloat16)
    out = gpu_multi(dst, c, q, split_blocks=split, window=window)
    Kd, Vd = orc.q4_dequant(img, tab, lens_np)
    ref = orc.attention_multi(Kd, Vd, bits(q), tab, lens_np, c.scale, window=window)
    assert max_err(out, ref) <= TOL


@pytest.mark.parametrize("n_h,k", [(32, 16), (64, 3), (32, 4)])
def test_multi_token_merge_many_pieces(n_h, k):
    """Long contexts beside empty, short and invalid (negative length)
    sequences, several query tokens: a (sequence, unit) pair is cut into many
    pieces that the row-group merge combines (64, 24 and 16 rows per unit);
    the invalid sequence's rows are NaN."""
    lens = [9000, 4000, 0, 40, 20]
    c = wl.make_case(1010 + k, len(lens), lens, n_h, 8, 128, "bf16", append=False, device=DEV)
    pool = new_pool(c)
    g = torch.Generator(device=DEV).manual_seed(k)
    q = torch.randn((c.batch, k, n_h, 128), generator=g, device=DEV).to(torch.bfloat16)
    bad = 4
    c.ctx_lens[bad] = -5
    out = gpu_multi(pool, c, q)
    good = [0, 1, 2, 3]
    tab, ctx = c.tables.cpu().numpy(), c.ctx_lens.cpu().numpy()
    ref = orc.attention_multi(bits(c.K), bits(c.V), bits(q)[good], tab[good], ctx[good], c.scale)
    assert np.all(np.isfinite(out[good]))
    assert max_err(out[good], ref) <= TOL
    assert np.all(np.isnan(out[bad]))


@pytest.mark.parametrize("k", [1, 3])
def test_int4_pool_over_4gib(k):
    """The same INT4 tiles in a small pool (its INT4 arrays span less than
    4 GiB: one buffer descriptor, 32-bit tile offsets) and at the far end of a
    4.4 GB pool (per-tile descriptors from 64-bit addresses): bitwise equal
    outputs on both schedules, for one query token (at most four query
    columns per kv head) and for three."""
    lens = [700, 37, 1500]
    c = int4_case(995 + k, lens, n_h=16, n_kv=8, d=128)
    c.append = False
    c.ctx_lens = c.seq_lens.clone()
    src, dst, img = int4_pools(c, len(lens))
    kv.kv_quantize_int4(dst, src, c.tables, c.seq_lens)
    nb_big = 210_000
    big = kv.KVPool(nb_big, c.n_kv, c.d, "int4", max_seqs=len(lens), device=DEV)
    assert big.nbytes > (1 << 32) + (1 << 26)  # the INT4 arrays alone span more than 4 GiB
    ids = torch.arange(c.num_blocks, device=DEV)
    moved = nb_big - 1 - ids  # block i of the small pool -> block nb_big - 1 - i
    for name in ["KQ", "KS", "KM", "VQ", "VS", "VM"]:
        getattr(big, name)[moved] = getattr(dst, name)[ids]
    big.KTAIL.copy_(dst.KTAIL)
    far = copy.copy(c)
    far.tables = torch.where(c.tables >= 0, nb_big - 1 - c.tables, c.tables)
    g = torch.Generator(device=DEV).manual_seed(40 + k)
    q = torch.randn((c.batch, k, c.n_h, 128), generator=g, device=DEV).to(torch.bfloat16)
    tab, lens_np = c.tables.cpu().numpy(), c.seq_lens.cpu().numpy()
    orc.q4_quantize_pool(img, bits(c.K), bits(c.V), tab, lens_np)
    Kd, Vd = orc.q4_dequant(img, tab, lens_np)
    ref = orc.attention_multi(Kd, Vd, bits(q), tab, lens_np, c.scale)
    for schedule, split in [(0, 0), (1, 40)]:
        a = gpu_multi(dst, c, q, split_blocks=split, schedule=schedule)
        b = gpu_multi(big, far, q, split_blocks=split, schedule=schedule)
        assert np.array_equal(a, b)
        assert max_err(a, ref) <= TOL
    del big


@pytest.mark.parametrize("dtype", ["f32", "bf16", "int4"])
@pytest.mark.parametrize("n_new", [1, 3, 16, 20])
def test_append_tokens_equals_sequential_appends(dtype, n_new):
    lens = [0, 5, 15, 16, 30, 47]
    n_kv, d = 2, 128
    pool_dtype = "bf16" if dtype == "int4" else dtype
    c = wl.make_case(990 + n_new, len(lens), lens, 4, n_kv, d, pool_dtype, num_blocks=40, append=False,
                     device=DEV, max_blocks=6)
    # tables with room for n_new more tokens: extend each row with unused ids
    need = [(L + n_new + 15) // 16 for L in lens]
    used = set(int(x) for x in c.tables.cpu().flatten() if x >= 0)
    free = [i for i in range(40) if i not in used]
    tab = c.tables.cpu().clone()
    for b, L in enumerate(lens):
        have = (L + 15) // 16
        for j in range(have, need[b]):
            tab[b, j] = free.pop()
    c.tables = tab.to(DEV)
    g = torch.Generator(device=DEV).manual_seed(n_new)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    kn = torch.randn((len(lens), n_new, n_kv, d), generator=g, device=DEV).to(tdt)
    vn = torch.randn((len(lens), n_new, n_kv, d), generator=g, device=DEV).to(tdt)
    lens_np = c.seq_lens.cpu().numpy()
    if dtype == "int4":
        src, dst, img = int4_pools(c, len(lens))
        kv.kv_quantize_int4(dst, src, c.tables, c.seq_lens)
        orc.q4_quantize_pool(img, bits(c.K), bits(c.V), tab.numpy(), lens_np)
        kv.kv_append_tokens(dst, kn, vn, c.tables, c.seq_lens)
        for t in range(n_new):
            orc.q4_append(img, bits(kn[:, t]), bits(vn[:, t]), tab.numpy(), lens_np + t)
        torch.cuda.synchronize()
        assert_img_equal(dst, img)
    else:
        pool = new_pool(c)
        kv.kv_append_tokens(pool, kn, vn, c.tables, c.seq_lens)
        torch.cuda.synchronize()
        K, V = bits(c.K), bits(c.V)
        for t in range(n_new):
            orc.append(K, V, bits(kn[:, t]), bits(vn[:, t]), tab.numpy(), lens_np + t)
        assert np.array_equal(ibits(bits(pool.K)), ibits(K)) and np.array_equal(ibits(bits(pool.V)), ibits(V))


# ---------------------------------------------------------------------------
# read-ceiling probe (measurement)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("pieces,at,workgroups", [(7, 6, 1), (7, 0, 0), (1001, 1000, 3), (4096, 2049, 2)])
def test_read_probe_reads_every_piece(pieces, at, workgroups):
    """A buffer of zeros with one word equal to the sink value, in piece `at`:
    the probe's XOR fold equals it only if that piece was read, and then the
    sink is written; with no such word the sink stays untouched."""
    buf = torch.zeros(pieces * 1024, dtype=torch.int32, device=DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv.kv_read_probe(buf, sink, workgroups)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    magic = np.array([0x9E3779B9], dtype=np.uint32).view(np.int32)[0]
    buf[at * 1024 + 517] = int(magic)
    kv.kv_read_probe(buf, sink, workgroups)
    torch.cuda.synchronize()
    assert int(sink.item()) == int(magic)
