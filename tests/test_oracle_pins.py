"""Pins of the oracle against what the pages and the mathematics fix.

None of these tests needs a GPU. They check the oracle (oracle/kvoracle.c)
against printed page values (tests/golden/), closed forms, invariants and
library routines, so that a dropped term, a wrong sign or index, or a
transposed operand in the oracle fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

from conftest import read_golden
import workloads as wl

BLOCK = 16


# ---------------------------------------------------------------------------
# helpers (test-side only: building pools and logical views)
# ---------------------------------------------------------------------------

def small_case(seed, lens, n_h, n_kv, d, dtype="f32", append=False, num_blocks=None, poison=True):
    c = wl.make_case(seed, len(lens), list(lens), n_h, n_kv, d, dtype, num_blocks=num_blocks,
                     append=append, poison=poison)
    return c


def host(c):
    return (wl.to_host_bits(c.K), wl.to_host_bits(c.V), wl.to_host_bits(c.q),
            c.tables.numpy(), c.ctx_lens.numpy())


def as_f64(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def logical(pool, tables, b, n):
    """[n][n_kv][d] view of sequence b's first n tokens (fancy indexing)."""
    idx = np.arange(n)
    return pool[tables[b, idx // BLOCK], :, idx % BLOCK, :]


def torch_attention(Kp, Vp, q, tables, ctx, scale, window=0):
    """Independent check: contiguous attention with torch.softmax in fp64."""
    Kf, Vf, qf = as_f64(Kp), as_f64(Vp), as_f64(q)
    B, n_h, d = qf.shape
    n_kv = Kf.shape[1]
    g = n_h // n_kv
    out = np.zeros((B, n_h, d))
    for b in range(B):
        n = int(ctx[b])
        s0 = max(0, n - window) if window else 0
        if n - s0 <= 0:
            continue
        k = torch.from_numpy(logical(Kf, tables, b, n)[s0:])    # [n][n_kv][d]
        v = torch.from_numpy(logical(Vf, tables, b, n)[s0:])
        for h in range(n_h):
            qh = torch.from_numpy(qf[b, h])
            w = torch.softmax((k[:, h // g, :] @ qh) * scale, dim=0)
            out[b, h] = (w @ v[:, h // g, :]).numpy()
    return out


# ---------------------------------------------------------------------------
# memory formula
# ---------------------------------------------------------------------------

UNITS = {"B": 1.0, "KiB": 1024.0, "GiB": 1024.0 ** 3, "GB": 1e9}


def test_memory_formula_matches_printed_sizes(orc):
    rows = read_golden("memory_budget.txt")
    assert len(rows) >= 8
    for label, L, T, dh, nkv, b, req, val, unit, tol, _src in rows:
        got = orc.kv_bytes(float(L), float(T), float(dh), float(nkv), float(b)) * float(req)
        assert abs(got / UNITS[unit] - float(val)) <= float(tol), (label, got)


def test_memory_formula_exact_bytes(orc):
    # exact integers behind the printed figures
    assert orc.kv_bytes(32, 2048, 128, 32, 2) == 1_073_741_824
    assert orc.kv_bytes(80, 2048, 128, 64, 2) == 5_368_709_120
    assert orc.kv_bytes(80, 2048, 128, 8, 2) == 671_088_640
    assert orc.kv_bytes(80, 2048, 128, 8, 0.5) == 167_772_160
    # GQA saves exactly n_h / n_kv
    assert orc.kv_bytes(80, 2048, 128, 64, 2) / orc.kv_bytes(80, 2048, 128, 8, 2) == 8.0


# ---------------------------------------------------------------------------
# scalar conversions
# ---------------------------------------------------------------------------

def _interesting_f32(n, seed):
    rng = np.random.default_rng(seed)
    x = np.concatenate([
        rng.standard_normal(n).astype(np.float32) * np.float32(10.0) ** rng.integers(-9, 6, n).astype(np.float32),
        np.array([0.0, -0.0, 65504.0, 65519.0, 65520.0, 70000.0, -65520.0, 2 ** -14, 2 ** -24, 2 ** -25,
                  3 * 2 ** -26, 2 ** -26, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 6.1e-5, 1e-8, np.inf, -np.inf],
                 dtype=np.float32),
    ])
    return x.astype(np.float32)


def test_f16_rounding_matches_numpy(orc):
    x = _interesting_f32(20000, 1)
    ref = x.astype(np.float16).view(np.uint16)
    got = orc.f32_to_f16_bits(x)
    assert np.array_equal(got, ref)


def test_f16_decode_matches_numpy(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = orc.f16_bits_to_f32(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_rounding_matches_torch(orc):
    x = _interesting_f32(20000, 2)
    x = x[np.isfinite(x)]
    extra = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 3.3895314e38, 3.39e38, 1e-40, -1e-42], dtype=np.float32)
    x = np.concatenate([x, extra])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.f32_to_bf16_bits(x)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def test_attention_closed_form(orc):
    """Two tokens, d = 2, scale 1, q = (1, 0), keys (0, 0) and (ln 3, 0):
    scores 0 and ln 3, weights 1/4 and 3/4; values (4, 0) and (0, 8) give
    exactly (1, 6)."""
    K = np.zeros((1, 1, BLOCK, 2))
    V = np.zeros((1, 1, BLOCK, 2))
    K[0, 0, 1] = [math.log(3.0), 0.0]
    V[0, 0, 0] = [4.0, 0.0]
    V[0, 0, 1] = [0.0, 8.0]
    q = np.array([[[1.0, 0.0]]])
    out = orc.attention(K, V, q, np.array([[0]]), np.array([2]), 1.0)
    assert np.allclose(out[0, 0], [1.0, 6.0], atol=1e-14, rtol=0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [((37, 50), 4, 2, 64), ((1, 16, 17, 33), 8, 8, 64),
                                   ((5, 31), 8, 1, 128), ((70,), 6, 2, 64)])
def test_attention_matches_torch_softmax(orc, dtype, shape):
    lens, n_h, n_kv, d = shape
    c = small_case(11, lens, n_h, n_kv, d, dtype)
    K, V, q, tab, ctx = host(c)
    got = orc.attention(K, V, q, tab, ctx, c.scale)
    ref = torch_attention(K, V, q, tab, ctx, c.scale)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_attention_one_token_returns_v(orc):
    c = small_case(3, (1, 1, 1), 4, 2, 64, "bf16")
    K, V, q, tab, ctx = host(c)
    out = orc.attention(K, V, q, tab, ctx, c.scale)
    Vf = as_f64(V)
    for b in range(3):
        for h in range(4):
            assert np.array_equal(out[b, h], Vf[tab[b, 0], h // 2, 0])


def test_attention_weights_sum_to_one(orc):
    c = small_case(4, (45, 9), 4, 2, 64, "f32")
    K, V, q, tab, ctx = host(c)
    ones = np.ones_like(V)
    out = orc.attention(K, ones, q, tab, ctx, c.scale)
    assert np.max(np.abs(out - 1.0)) < 1e-14


def test_attention_identical_keys_give_mean_value(orc):
    c = small_case(5, (29,), 2, 1, 64, "f32", poison=False)
    K, V, q, tab, ctx = host(c)
    K[:] = K[tab[0, 0], :, 0:1, :]          # every key equal to the first
    out = orc.attention(K, V, q, tab, ctx, c.scale)
    mean = logical(as_f64(V), tab, 0, 29)[:, 0, :].mean(axis=0)
    assert np.max(np.abs(out[0] - mean)) < 1e-13


def test_attention_key_shift_and_value_offset(orc):
    c = small_case(6, (40, 23), 4, 2, 64, "f32", poison=False)
    K, V, q, tab, ctx = host(c)
    K64, V64 = as_f64(K), as_f64(V)
    base = orc.attention(K64, V64, q, tab, ctx, c.scale)
    u = np.random.default_rng(0).standard_normal(64)
    shifted = orc.attention(K64 + u, V64, q, tab, ctx, c.scale)    # every score moves by q.u
    assert np.max(np.abs(shifted - base)) < 1e-12
    offset = orc.attention(K64, V64 + 2.5, q, tab, ctx, c.scale)
    assert np.max(np.abs(offset - (base + 2.5))) < 1e-12


def test_gqa_equals_mha_with_replicated_kv(orc):
    c = small_case(7, (33, 48), 8, 2, 64, "bf16", poison=False)
    K, V, q, tab, ctx = host(c)
    g = 4
    Km = np.repeat(K, g, axis=1)            # kv head h -> heads h*g .. h*g+g-1
    Vm = np.repeat(V, g, axis=1)
    gqa = orc.attention(K, V, q, tab, ctx, c.scale)
    mha = orc.attention(Km, Vm, q, tab, ctx, c.scale)
    assert np.array_equal(gqa, mha)


def test_mqa_each_head_is_single_head_attention(orc):
    c = small_case(8, (20,), 4, 1, 64, "f32", poison=False)
    K, V, q, tab, ctx = host(c)
    mqa = orc.attention(K, V, q, tab, ctx, c.scale)
    for h in range(4):
        one = orc.attention(K, V, np.ascontiguousarray(q[:, h:h + 1]), tab, ctx, c.scale)
        assert np.array_equal(mqa[:, h], one[:, 0])


def test_query_groups_are_contiguous(orc):
    """Heads 0,1 read kv head 0 and heads 2,3 read kv head 1 (n_h 4, n_kv 2)."""
    c = small_case(9, (18,), 4, 2, 64, "f32", poison=False)
    K, V, q, tab, ctx = host(c)
    V[:, 0] = 1.0
    V[:, 1] = -1.0
    out = orc.attention(K, V, q, tab, ctx, c.scale)
    assert np.all(out[0, :2] == 1.0) and np.all(out[0, 2:] == -1.0)


def test_block_permutation_invariance(orc):
    c = small_case(10, (37, 50, 16), 4, 2, 64, "bf16", num_blocks=20)
    K, V, q, tab, ctx = host(c)
    base = orc.attention(K, V, q, tab, ctx, c.scale)
    perm = np.random.default_rng(1).permutation(K.shape[0])   # old id -> new id
    K2 = np.empty_like(K)
    V2 = np.empty_like(V)
    K2[perm] = K
    V2[perm] = V
    tab2 = np.where(tab >= 0, perm[np.maximum(tab, 0)], -1).astype(np.int32)
    moved = orc.attention(K2, V2, q, tab2, ctx, c.scale)
    assert np.array_equal(base, moved)


def test_empty_context_gives_zero(orc):
    c = small_case(12, (0, 5), 4, 2, 64, "f32")
    K, V, q, tab, ctx = host(c)
    tab = np.where(tab < 0, 0, tab).astype(np.int32)
    out = orc.attention(K, V, q, tab, ctx, c.scale)
    assert np.all(out[0] == 0.0) and np.all(np.isfinite(out[1]))


def test_large_scores_do_not_overflow(orc):
    c = small_case(13, (30,), 2, 1, 64, "f32", poison=False)
    K, V, q, tab, ctx = host(c)
    out = orc.attention(K * 1000.0, V, q, tab, ctx, c.scale)
    assert np.all(np.isfinite(out))
    ref = torch_attention(K * 1000.0, V, q, tab, ctx, c.scale)
    assert np.max(np.abs(out - ref)) < 1e-10


@pytest.mark.parametrize("window", [1, 7, 16, 17, 100])
def test_window_attends_last_tokens(orc, window):
    c = small_case(14, (40, 5), 4, 2, 64, "f32")
    K, V, q, tab, ctx = host(c)
    got = orc.attention(K, V, q, tab, ctx, c.scale, window=window)
    ref = torch_attention(K, V, q, tab, ctx, c.scale, window=window)
    assert np.max(np.abs(got - ref)) < 1e-12
    if window == 1:
        Vf = as_f64(V)
        last = logical(Vf, tab, 0, 40)[39]
        assert np.array_equal(got[0, 0], last[0])
    if window >= 40:
        assert np.array_equal(got, orc.attention(K, V, q, tab, ctx, c.scale))


# ---------------------------------------------------------------------------
# append
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_append_writes_exactly_one_slot(orc, dtype):
    c = small_case(20, (37, 50, 0, 15, 16), 4, 2, 64, dtype, append=True, num_blocks=24)
    K, V, q, tab, ctx = host(c)
    kn, vn = wl.to_host_bits(c.k_new), wl.to_host_bits(c.v_new)
    lens = c.seq_lens.numpy()
    K2, V2 = K.copy(), V.copy()
    orc.append(K2, V2, kn, vn, tab, lens)
    itype = np.uint32 if dtype == "f32" else np.uint16
    dk = K2.view(itype) != K.view(itype)
    dv = V2.view(itype) != V.view(itype)
    assert dk.sum() <= len(lens) * 2 * 64 and dv.sum() <= len(lens) * 2 * 64
    for b, L in enumerate(lens):
        p, t = tab[b, L // BLOCK], L % BLOCK
        assert np.array_equal(K2[p, :, t, :].view(itype), kn[b].view(itype))
        assert np.array_equal(V2[p, :, t, :].view(itype), vn[b].view(itype))
    # everything outside the written slots is unchanged, NaN poison included
    mask = np.ones(K.shape[:3], dtype=bool)
    for b, L in enumerate(lens):
        mask[tab[b, L // BLOCK], :, L % BLOCK] = False
    assert np.array_equal(K2.view(itype)[mask], K.view(itype)[mask])
    assert np.array_equal(V2.view(itype)[mask], V.view(itype)[mask])


def test_append_then_attend_one_token_returns_new_value(orc):
    c = small_case(21, (0, 0), 4, 2, 64, "bf16", append=True)
    K, V, q, tab, ctx = host(c)
    kn, vn = wl.to_host_bits(c.k_new), wl.to_host_bits(c.v_new)
    orc.append(K, V, kn, vn, tab, c.seq_lens.numpy())
    out = orc.attention(K, V, q, tab, ctx, c.scale)
    for b in range(2):
        for h in range(4):
            assert np.array_equal(out[b, h], as_f64(vn[b, h // 2]))


def test_append_then_attend_matches_torch(orc):
    c = small_case(22, (37, 50), 4, 2, 64, "f32", append=True, num_blocks=16)
    K, V, q, tab, ctx = host(c)
    orc.append(K, V, wl.to_host_bits(c.k_new), wl.to_host_bits(c.v_new), tab, c.seq_lens.numpy())
    got = orc.attention(K, V, q, tab, ctx, c.scale)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - torch_attention(K, V, q, tab, ctx, c.scale))) < 1e-12


# ---------------------------------------------------------------------------
# INT4
# ---------------------------------------------------------------------------

def test_int4_golden_groups(orc):
    rows = read_golden("int4_groups.txt")
    assert len(rows) == 13
    for label, xs, codes, s16, m16, _why in rows:
        x = np.array([float.fromhex(v) if "0x" in v else float(v) for v in xs.split(",")], dtype=np.float32)
        got_c, got_s, got_m = orc.q4_group(x)
        assert list(got_c) == [int(v) for v in codes.split(",")], label
        assert got_s == int(s16, 16), label
        assert got_m == int(m16, 16), label


def test_int4_error_bound_and_range(orc):
    """Codes lie in [0, 15] at every magnitude, and where the stored s and min
    are finite the reconstruction error obeys the closed-form bound. Scales
    from 10^-7.5 (fp16 subnormal s and min: the clamp binds in many groups)
    to 10^6 (fp16 overflow)."""
    rng = np.random.default_rng(5)
    clamped = 0
    for trial in range(600):
        n = 16 if trial % 2 else 128
        x32 = (rng.standard_normal(n) * 10.0 ** rng.uniform(-7.5, 6)).astype(np.float32)
        xb = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        x = as_f64(xb)
        codes, s16, m16 = orc.q4_group(xb)
        assert codes.max() <= 15 and codes.min() >= 0, trial
        s = float(orc.f16_bits_to_f32(np.array([s16]))[0])
        m = float(orc.f16_bits_to_f32(np.array([m16]))[0])
        if not (np.isfinite(s) and np.isfinite(m)) or s == 0.0:
            continue
        mn, mx = x.min(), x.max()
        s32 = float(np.float32(np.float32(mx) - np.float32(mn)) / np.float32(15.0))
        xhat = m + codes.astype(np.float64) * s
        bound = max(s / 2, abs(mn - m) + 15 * abs(s32 - s)) + 1e-6 * max(abs(mn), abs(mx))
        assert np.max(np.abs(x - xhat)) <= bound, trial
        # an exact quotient of 15.5 or more, or -0.5 or less: a clamped code
        v = (x - m) / s
        clamped += int(np.any(v >= 15.5) or np.any(v <= -0.5))
    assert clamped >= 10  # the draw reaches the clamp regime (17 groups with this seed)


def test_int4_requantizing_grid_values_is_stable(orc):
    rng = np.random.default_rng(6)
    for _ in range(50):
        x = (rng.standard_normal(16) * 3).astype(np.float32)
        codes, s16, m16 = orc.q4_group(x)
        if codes.min() != 0 or codes.max() != 15:
            continue
        s = orc.f16_bits_to_f32(np.array([s16]))[0]
        m = orc.f16_bits_to_f32(np.array([m16]))[0]
        xhat = (m + codes.astype(np.float32) * s).astype(np.float32)
        c2, s2, m2 = orc.q4_group(xhat)
        assert np.array_equal(c2, codes) and s2 == s16 and m2 == m16


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def test_int4_group_orientation(orc):
    """K groups run over tokens (per channel), V groups over channels (per
    token): a K block whose channels are constant over tokens and a V block
    whose tokens are constant over channels come back exactly."""
    n_kv, d, nb = 2, 64, 3
    rng = np.random.default_rng(7)
    chan_vals = rng.integers(-64, 64, size=(n_kv, d)) / 8.0        # fp16/bf16-exact
    tok_vals = rng.integers(-64, 64, size=(nb, n_kv, BLOCK)) / 8.0
    K = np.broadcast_to(chan_vals[None, :, None, :], (nb, n_kv, BLOCK, d))
    V = np.broadcast_to(tok_vals[..., None], (nb, n_kv, BLOCK, d))
    Kb, Vb = _bf16(K), _bf16(V)
    tables = np.array([[0, 1, 2]], dtype=np.int32)
    lens = np.array([48])
    img = orc.Q4Image(nb, n_kv, d, 1)
    orc.q4_quantize_pool(img, Kb, Vb, tables, lens)
    Kd, Vd = orc.q4_dequant(img, tables, lens)
    assert np.array_equal(Kd, K) and np.array_equal(Vd, V)
    assert np.all(img.ks == 0) and np.all(img.vs == 0)


def test_int4_nibble_packing(orc):
    """Channel 2c goes to the low nibble of byte c, channel 2c+1 to the high."""
    d = 16
    v = np.zeros((1, 1, BLOCK, d), dtype=np.float32)
    v[0, 0, 0] = np.arange(16) * 1.5          # codes 0..15 along the channels
    img = orc.Q4Image(1, 1, d, 1)
    orc.q4_quantize_pool(img, _bf16(np.zeros_like(v)), _bf16(v), np.array([[0]]), np.array([1]))
    assert list(img.vq[0, 0, 0]) == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]


@pytest.mark.parametrize("n_tokens", [16, 40, 47, 48])
def test_int4_append_token_by_token_equals_bulk(orc, n_tokens):
    n_kv, d = 2, 64
    nblk = (n_tokens + 15) // 16
    rng = np.random.default_rng(n_tokens)
    toks_k = _bf16(rng.standard_normal((n_tokens, n_kv, d)) * 2)
    toks_v = _bf16(rng.standard_normal((n_tokens, n_kv, d)))
    tables = np.array([rng.permutation(8)[:nblk]], dtype=np.int32)
    # bulk: lay the tokens into a bf16 pool, then convert
    Kb = np.zeros((8, n_kv, BLOCK, d), dtype=np.uint16)
    Vb = np.zeros_like(Kb)
    for j in range(n_tokens):
        Kb[tables[0, j // 16], :, j % 16] = toks_k[j]
        Vb[tables[0, j // 16], :, j % 16] = toks_v[j]
    bulk = orc.Q4Image(8, n_kv, d, 1)
    orc.q4_quantize_pool(bulk, Kb, Vb, tables, np.array([n_tokens]))
    inc = orc.Q4Image(8, n_kv, d, 1)
    for j in range(n_tokens):
        orc.q4_append(inc, toks_k[j][None], toks_v[j][None], tables, np.array([j]))
    for name in ["kq", "ks", "km", "vq", "vs", "vm"]:
        assert np.array_equal(getattr(inc, name), getattr(bulk, name)), name
    r = n_tokens % 16
    assert np.array_equal(inc.kt[:, :, :r], bulk.kt[:, :, :r])


def test_int4_attention_on_grid_values_equals_bf16_attention(orc):
    """Values already on each group's INT4 grid dequantize exactly, so
    attention over the INT4 image equals attention over the bf16 pool."""
    n_kv, d, n_h = 2, 64, 4
    rng = np.random.default_rng(8)
    nb = 4
    # K per channel on the grid {m + k s}: pick per-(block, head, channel) m, s
    m = rng.integers(-8, 8, size=(nb, n_kv, 1, d)) / 4.0
    s = rng.integers(1, 4, size=(nb, n_kv, 1, d)) / 8.0
    codes = rng.integers(0, 16, size=(nb, n_kv, BLOCK, d))
    codes[:, :, 0, :] = 0
    codes[:, :, 1, :] = 15
    K = m + codes * s
    mv = rng.integers(-8, 8, size=(nb, n_kv, BLOCK, 1)) / 4.0
    sv = rng.integers(1, 4, size=(nb, n_kv, BLOCK, 1)) / 8.0
    cv = rng.integers(0, 16, size=(nb, n_kv, BLOCK, d))
    cv[..., 0] = 0
    cv[..., 1] = 15
    V = mv + cv * sv
    Kb, Vb = _bf16(K), _bf16(V)
    assert np.array_equal(as_f64(Kb), K) and np.array_equal(as_f64(Vb), V)
    tables = np.array([[2, 0], [1, 3]], dtype=np.int32)
    lens = np.array([32, 32])
    img = orc.Q4Image(nb, n_kv, d, 2)
    orc.q4_quantize_pool(img, Kb, Vb, tables, lens)
    Kd, Vd = orc.q4_dequant(img, tables, lens)
    q = _bf16(rng.standard_normal((2, n_h, d)))
    a = orc.attention(Kd, Vd, q, tables, lens, 0.125)
    b = orc.attention(Kb, Vb, q, tables, lens, 0.125)
    assert np.array_equal(a, b)


def test_int4_per_channel_beats_per_token_on_outlier_keys(orc):
    """Direction of the KVQuant observation on synthetic outlier keys
    (information: 4 of 128 channels scaled x10)."""
    rng = np.random.default_rng(9)
    K = rng.standard_normal((BLOCK, 128)).astype(np.float32)
    K[:, [3, 40, 77, 120]] *= 10
    Kb = _bf16(K)
    x = as_f64(Kb)

    def mse(groups_axis):
        err = 0.0
        for i in range(x.shape[groups_axis]):
            grp = np.ascontiguousarray(Kb[:, i] if groups_axis == 1 else Kb[i])
            codes, s16, m16 = orc.q4_group(grp)
            s = orc.f16_bits_to_f32(np.array([s16]))[0]
            mm = orc.f16_bits_to_f32(np.array([m16]))[0]
            ref = x[:, i] if groups_axis == 1 else x[i]
            err += np.sum((mm + codes * np.float64(s) - ref) ** 2)
        return err / x.size

    assert mse(1) < mse(0)


# ---------------------------------------------------------------------------
# RoPE re-rotation
# ---------------------------------------------------------------------------

def test_rope_golden_angles(orc):
    rows = read_golden("rope_angles.txt")
    for label, i, delta, style, xin, xout in rows:
        i, delta, style = int(i), int(delta), int(style)
        K = np.zeros((1, 1, BLOCK, 128), dtype=np.float32)
        c0, c1 = (2 * i, 2 * i + 1) if style == 0 else (i, i + 64)
        x, y = [float(v) for v in xin.split(",")]
        K[0, 0, 0, c0], K[0, 0, 0, c1] = x, y
        orc.rope_rerotate(K, np.array([0]), 0, 1, delta, 10000.0, style)
        ex, ey = [float(v) for v in xout.split(",")]
        assert abs(K[0, 0, 0, c0] - ex) <= 2e-7 and abs(K[0, 0, 0, c1] - ey) <= 2e-7, label
        others = np.delete(K[0, 0, 0], [c0, c1])
        assert np.all(others == 0.0), label


def test_rope_zero_offset_is_identity(orc):
    c = small_case(30, (64,), 4, 4, 128, "bf16", poison=False)
    K = wl.to_host_bits(c.K)
    K2 = K.copy()
    orc.rope_rerotate(K2, c.tables.numpy()[0], 0, 64, 0, 10000.0, 0)
    assert np.array_equal(K, K2)


def test_rope_relative_position_property(orc):
    rng = np.random.default_rng(10)
    for style in (0, 1):
        q = rng.standard_normal(128)
        k = rng.standard_normal(128)
        m, n, delta = 37, 5, 1234
        a = orc.rope_rotate_f64(q, m, 10000.0, style) @ orc.rope_rotate_f64(k, n, 10000.0, style)
        b = orc.rope_rotate_f64(q, m + delta, 10000.0, style) @ orc.rope_rotate_f64(k, n + delta, 10000.0, style)
        assert abs(a - b) <= 1e-11 * (1 + abs(a))
        # composition and norm preservation
        r2 = orc.rope_rotate_f64(orc.rope_rotate_f64(k, 300, 10000.0, style), 4000, 10000.0, style)
        r1 = orc.rope_rotate_f64(k, 4300, 10000.0, style)
        assert np.max(np.abs(r1 - r2)) < 1e-11
        assert abs(np.linalg.norm(r1) - np.linalg.norm(k)) < 1e-12


@pytest.mark.parametrize("style", [0, 1])
def test_rope_bf16_within_one_ulp_of_exact_rotation(orc, style):
    c = small_case(31, (48,), 2, 2, 128, "bf16", poison=False)
    K = wl.to_host_bits(c.K)
    tab = c.tables.numpy()[0]
    K2 = K.copy()
    delta = 9876
    orc.rope_rerotate(K2, tab[1:3], 3, 20, delta, 10000.0, style)   # tokens 3..22 of blocks 1, 2
    Kf, K2f = as_f64(K), as_f64(K2)
    chunk = [(tab[1 + (3 + j) // 16], (3 + j) % 16) for j in range(20)]
    for p, t in chunk:
        for h in range(2):
            exact = orc.rope_rotate_f64(Kf[p, h, t], delta, 10000.0, style)
            ulp = np.maximum(np.abs(exact), 1e-30)
            ulp = 2.0 ** (np.floor(np.log2(ulp)) - 7)
            assert np.all(np.abs(K2f[p, h, t] - exact) <= ulp * 1.01 + 1e-6)
    touched = np.zeros(K.shape[:3], dtype=bool)
    for p, t in chunk:
        touched[p, :, t] = True
    assert np.array_equal(K2[~touched], K[~touched])


@pytest.mark.parametrize("n_tokens", [1, 21, 40])
def test_int4_partial_block_keys_read_back_exactly(orc, n_tokens):
    """Keys of a block that is not yet full stay in bf16, so they read back
    bit-exactly; keys of full blocks come back within their group's step."""
    n_kv, d = 2, 64
    rng = np.random.default_rng(40 + n_tokens)
    Kb = _bf16(rng.standard_normal((4, n_kv, BLOCK, d)))
    Vb = _bf16(rng.standard_normal((4, n_kv, BLOCK, d)))
    tables = np.array([[3, 1, 0]], dtype=np.int32)
    lens = np.array([n_tokens])
    img = orc.Q4Image(4, n_kv, d, 2)
    orc.q4_quantize_pool(img, Kb, Vb, tables, lens, slots=np.array([1]))
    Kd, _ = orc.q4_dequant(img, tables, lens, slots=np.array([1]))
    full = n_tokens // 16
    for j in range(full * 16, n_tokens):
        p, t = tables[0, j // 16], j % 16
        assert np.array_equal(Kd[p, :, t], as_f64(Kb[p, :, t]))
    for j in range(full * 16):
        p, t = tables[0, j // 16], j % 16
        assert not np.array_equal(Kd[p, :, t], as_f64(Kb[p, :, t]))   # really quantized
        assert np.max(np.abs(Kd[p, :, t] - as_f64(Kb[p, :, t]))) < 0.5
    assert np.all(img.kt[0] == 0)            # slot 0 untouched: the tail lives in slot 1


# ---------------------------------------------------------------------------
# block copies (copy-on-reuse, offload / restore)
# ---------------------------------------------------------------------------

def test_block_copy_gather_scatter_round_trip(orc):
    rng = np.random.default_rng(50)
    K = rng.integers(0, 65535, size=(12, 2, 16, 64), dtype=np.uint16)
    V = rng.integers(0, 65535, size=(12, 2, 16, 64), dtype=np.uint16)
    ks = rng.integers(0, 65535, size=(12, 2, 64), dtype=np.uint16)   # a region of another block size
    K0, V0, ks0 = K.copy(), V.copy(), ks.copy()
    blocks = np.array([7, 2, 11, 0])
    buf = orc.gather_blocks([K, V, ks], blocks)
    per = (2 * 16 * 64 * 2) * 2 + 2 * 64 * 2
    assert buf.size == 4 * per
    # packed block i: K slice, then V slice, then ks slice, each equal to the source block
    for i, b in enumerate(blocks):
        seg = buf[i * per:(i + 1) * per]
        assert np.array_equal(seg[:4096].view(np.uint16).reshape(2, 16, 64), K[b])
        assert np.array_equal(seg[4096:8192].view(np.uint16).reshape(2, 16, 64), V[b])
        assert np.array_equal(seg[8192:].view(np.uint16).reshape(2, 64), ks[b])
    # scatter into other blocks, then the copies equal the originals
    dst = np.array([1, 3, 5, 9])
    orc.scatter_blocks([K, V, ks], dst, buf)
    for s_, d_ in zip(blocks, dst):
        assert np.array_equal(K[d_], K0[s_]) and np.array_equal(V[d_], V0[s_]) and np.array_equal(ks[d_], ks0[s_])
    untouched = [b for b in range(12) if b not in dst]
    assert np.array_equal(K[untouched], K0[untouched])


def test_block_copy_in_pool(orc):
    rng = np.random.default_rng(51)
    K = rng.standard_normal((10, 2, 16, 64)).astype(np.float32)
    V = rng.standard_normal((10, 2, 16, 64)).astype(np.float32)
    K0, V0 = K.copy(), V.copy()
    orc.copy_blocks([K, V], [4, 8], [0, 9])
    assert np.array_equal(K[0], K0[4]) and np.array_equal(K[9], K0[8])
    assert np.array_equal(V[0], V0[4]) and np.array_equal(V[9], V0[8])
    assert np.array_equal(K[1:9], K0[1:9])


# ---------------------------------------------------------------------------
# several query tokens per sequence
# ---------------------------------------------------------------------------

def torch_attention_multi(Kp, Vp, q, tables, ctx, scale, window=0):
    """Independent check: contiguous attention with an explicit causal mask."""
    Kf, Vf, qf = as_f64(Kp), as_f64(Vp), as_f64(q)
    B, k, n_h, d = qf.shape
    g = n_h // Kf.shape[1]
    out = np.zeros((B, k, n_h, d))
    for b in range(B):
        n = int(ctx[b])
        if n == 0:
            continue
        kk = torch.from_numpy(logical(Kf, tables, b, n))
        vv = torch.from_numpy(logical(Vf, tables, b, n))
        pos = torch.arange(n)
        for i in range(k):
            P = n - k + i
            allowed = (pos <= P) & ((pos > P - window) if window else torch.ones(n, dtype=torch.bool))
            if not bool(allowed.any()):
                continue
            for h in range(n_h):
                s = (kk[:, h // g, :] @ torch.from_numpy(qf[b, i, h])) * scale
                w = torch.softmax(s.masked_fill(~allowed, float("-inf")), dim=0)
                out[b, i, h] = (w @ vv[:, h // g, :]).numpy()
    return out


def _multi_q(c, k, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((c.batch, k, c.n_h, c.d)).astype(np.float32)
    return _bf16(q) if c.dtype == "bf16" else q


@pytest.mark.parametrize("k,window", [(1, 0), (3, 0), (4, 0), (5, 7), (16, 0)])
def test_multi_token_matches_torch_causal(orc, k, window):
    c = small_case(60, (3, 16, 40, 77), 8, 2, 64, "bf16", poison=False)
    K, V, _, tab, ctx = host(c)
    q = _multi_q(c, k, 61)
    got = orc.attention_multi(K, V, q, tab, ctx, c.scale, window=window)
    ref = torch_attention_multi(K, V, q, tab, ctx, c.scale, window=window)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_multi_token_last_query_is_decode_and_causality(orc):
    c = small_case(62, (20, 33, 50), 4, 2, 64, "f32", poison=False)
    K, V, _, tab, ctx = host(c)
    k = 4
    q = _multi_q(c, k, 63)
    multi = orc.attention_multi(K, V, q, tab, ctx, c.scale)
    # the last query token sees the whole cache: exactly the decode attention
    dec = orc.attention(K, V, np.ascontiguousarray(q[:, -1]), tab, ctx, c.scale)
    assert np.array_equal(multi[:, -1], dec)
    # query i is the decode attention over the first ctx - k + i + 1 tokens
    for i in range(k):
        dec_i = orc.attention(K, V, np.ascontiguousarray(q[:, i]), tab, ctx - k + i + 1, c.scale)
        assert np.array_equal(multi[:, i], dec_i)
    # changing a later token does not change an earlier query's output
    K2 = K.copy()
    p_last = tab[0, (ctx[0] - 1) // 16]
    K2[p_last, :, (ctx[0] - 1) % 16, :] += 5.0
    multi2 = orc.attention_multi(K2, V, q, tab, ctx, c.scale)
    assert np.array_equal(multi2[0, :k - 1], multi[0, :k - 1])
    assert not np.array_equal(multi2[0, k - 1], multi[0, k - 1])


# ---------------------------------------------------------------------------
# CacheBlend token selection
# ---------------------------------------------------------------------------

def test_deviation_definition(orc):
    rng = np.random.default_rng(70)
    # quarter-integers: every offset below is exact in fp32
    K = (rng.integers(-16, 16, (6, 2, 16, 64)) / 4).astype(np.float32)
    V = (rng.integers(-16, 16, (6, 2, 16, 64)) / 4).astype(np.float32)
    tables = np.array([[4, 1, 5], [0, 2, 3]])
    # rows: sequence 0 positions 3..22, then sequence 1 positions 40, 7
    rs = np.array([0] * 20 + [1, 1])
    rp = np.concatenate([3 + np.arange(20), [40, 7]])
    blk = tables[rs, rp // 16]
    pre_k, pre_v = K[blk, :, rp % 16, :], V[blk, :, rp % 16, :]
    # recomputed = precomputed: deviation 0; known offsets give known values
    assert np.all(orc.deviation(K, V, tables, rs, rp, pre_k, pre_v) == 0.0)
    k_re, v_re = pre_k.copy(), pre_v.copy()
    k_re[7] += 0.5                                         # 2 heads x 64 channels of 0.25
    v_re[11, 1, 3] -= 3.0                                  # one element of 9
    v_re[21, 0, 0] += 1.0                                  # sequence 1, position 7: one element of 1
    dev = orc.deviation(K, V, tables, rs, rp, k_re, v_re)
    assert dev[7] == 2 * 64 * 0.25 and dev[11] == 9.0 and dev[21] == 1.0
    assert np.count_nonzero(dev) == 3
    # a subset of the rows, in another order, gives the same values
    ids = np.array([21, 11, 7, 2])
    assert np.array_equal(orc.deviation(K, V, tables, rs[ids], rp[ids], k_re[ids], v_re[ids]), dev[ids])
    # the same row compared with another token's cache entry is not zero
    assert orc.deviation(K, V, tables, [0], [4], pre_k[:1], pre_v[:1])[0] > 0


def test_deviation_bf16_exact_case(orc):
    """bf16 pool: differences of small integers, squared and summed, are exact."""
    rng = np.random.default_rng(72)
    Kf = rng.integers(-8, 8, (3, 4, 16, 32)).astype(np.float32)
    Vf = rng.integers(-8, 8, (3, 4, 16, 32)).astype(np.float32)
    K, V = orc.f32_to_bf16_bits(Kf), orc.f32_to_bf16_bits(Vf)
    tables = np.array([[2, 0, 1]])
    rp = np.array([0, 17, 33, 47])
    blk = tables[0, rp // 16]
    dk = rng.integers(-3, 4, (4, 4, 32)).astype(np.float32)
    dv = rng.integers(-3, 4, (4, 4, 32)).astype(np.float32)
    k_re = orc.f32_to_bf16_bits(Kf[blk, :, rp % 16, :] + dk)
    v_re = orc.f32_to_bf16_bits(Vf[blk, :, rp % 16, :] + dv)
    dev = orc.deviation(K, V, tables, [0] * 4, rp, k_re, v_re)
    for i in range(4):                                     # integer sum of squares, counted by hand
        want = sum(int(x) ** 2 for x in dk[i].ravel()) + sum(int(x) ** 2 for x in dv[i].ravel())
        assert dev[i] == want


def test_topk_selection(orc):
    v = np.array([0.5, 3.0, 1.0, 3.0, -2.0, 7.0, 1.0])
    assert list(orc.topk(v, 3)) == [1, 3, 5]              # 7, then the two 3s
    assert list(orc.topk(v, 2)) == [1, 5]                 # tie between rows 1 and 3: the lower wins
    assert list(orc.topk(v, 5)) == [1, 2, 3, 5, 6]
    assert list(orc.topk(v, 0)) == []
    assert list(orc.topk(v, 99)) == list(range(7))
    rng = np.random.default_rng(71)
    x = rng.standard_normal(1000)
    sel = orc.topk(x, 150)
    ref = np.sort(np.argsort(-x, kind="stable")[:150])    # numpy's stable sort as the independent check
    assert np.array_equal(sel, ref)
    # ties in bulk: small integers; brute force over every k on a tiny input
    t = rng.integers(0, 4, 40).astype(np.float64)
    for k in range(41):
        order = sorted(range(40), key=lambda i: (-t[i], i))
        assert list(orc.topk(t, k)) == sorted(order[:k])
    # signed zeros tie; infinities order at the ends
    z = np.array([0.0, -0.0, np.inf, -np.inf, -0.0, 1.0])
    assert list(orc.topk(z, 3)) == [0, 2, 5]
    assert list(orc.topk(z, 5)) == [0, 1, 2, 4, 5]


def test_recompute_ratio(orc):
    # loading a layer takes as long as recomputing 40 % of 1000 tokens
    assert abs(orc.recompute_ratio(400.0, 1.0, 1000) - 0.4) < 1e-15
    # a fast load hides little: the 15 % floor applies
    assert orc.recompute_ratio(10.0, 1.0, 1000) == 0.15
    # a slow load could hide more than everything: capped at 1
    assert orc.recompute_ratio(5000.0, 1.0, 1000) == 1.0


def test_recompute_count(orc):
    assert orc.recompute_count(0.15, 1000) == 150
    assert orc.recompute_count(0.15, 7) == 2              # 1.05 rounds up: never below the ratio
    assert orc.recompute_count(0.5, 4) == 2
    assert orc.recompute_count(1.0, 33) == 33
    assert orc.recompute_count(0.0, 33) == 0
    assert orc.recompute_count(0.15, 0) == 0
    for n in range(1, 300):                                # the count never falls below ratio * n
        c = orc.recompute_count(0.15, n)
        assert c >= 0.15 * n - 1e-12 and c - 1 < 0.15 * n


# KVSYS "어텐션 윈도우 크기": the page's own example, max_attention_window =
# [4096, 256], makes the 1st, 3rd and 5th layers full attention and the 2nd,
# 4th and 6th limited to 256 tokens; a one-entry list covers every layer.
def test_layer_window_page_example(orc):
    assert [orc.layer_window([4096, 256], layer) for layer in range(6)] == [4096, 256, 4096, 256, 4096, 256]
    assert [orc.layer_window([4096], layer) for layer in range(5)] == [4096] * 5
    assert [orc.layer_window([7, 8, 9], layer) for layer in range(8)] == [7, 8, 9, 7, 8, 9, 7, 8]


# KVSYS "제한된 어텐션 윈도우 크기": blocks that no later query can attend are
# released. Brute force: the later queries of a sequence holding L tokens sit
# at positions L, L + 1, ...; each attends the last `window` tokens up to
# itself (all tokens for window 0). The released count is the first block any
# of them attends (every block from there on is attended by some query).
@pytest.mark.parametrize("window", [0, 1, 2, 15, 16, 17, 31, 32, 33, 64, 100, 1000])
def test_window_released_brute_force(orc, window):
    rng = np.random.default_rng(77 + window)
    lens = [int(x) for x in rng.integers(0, 300, 60)] + [0, 1, 15, 16, 17, 31, 32, 33, 999, -1, -500]
    got = orc.window_released(lens, window)
    for L, g in zip(lens, got):
        if L < 0:
            assert g == -1
            continue
        attended = set()
        for p in range(L, L + 40):
            lo = 0 if window == 0 else max(0, p + 1 - window)
            attended |= {t // 16 for t in range(lo, p + 1)}
        assert g == min(attended), (L, window)
