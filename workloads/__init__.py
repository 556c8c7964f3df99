"""Seeded synthetic inputs for the paged decode-attention path.

This module only draws inputs: pool contents, block tables, lengths, queries,
new tokens, outlier channels and rotation offsets. It holds none of the
method's arithmetic (no attention, quantization or rotation), so both the HIP
path and the oracle may take their inputs from it.

Everything is drawn with ``torch.Generator`` seeded per tensor kind, on the
device the caller names. Values on one device are reproducible for a seed;
the oracle always receives a host copy of the very tensors the GPU used.

Workloads (LLaMA-shaped decode layers; no weights or real activations exist
here, so N(0,1) data stands in for them):
  tiny            2 seqs, lengths 37 and 50, 4 q heads / 2 kv heads, d_h 64,
                  fp32, 16-block pool
  llama3_8b       64 seqs, lengths U{512..4096}, 32/8 heads, d_h 128, bf16,
                  pool = total blocks + 10 %
  llama2_70b      256 seqs, length 2048, 64/8 heads, d_h 128, bf16, pool exact
  kvquant_int4    llama3_8b shapes; K has 4 of 128 channels per kv head x10
  long_shared     8 seqs x 32768 tokens, 32/32 heads, d_h 128, bf16; the first
                  16384 tokens of every sequence share physical blocks; a
                  4096-token chunk of that prefix is re-rotated by a seeded
                  offset in [1, 16384]
  blend_select    16 requests x 8192 reused tokens, 8 kv heads, d_h 128,
                  bf16 (LLaMA-3-8B KV shape): recomputed K/V rows for every
                  reused token are the cached rows plus N(0, sigma_t^2) noise
                  with sigma_t^2 ~ U(0, 1) per token (a near-linear deviation
                  CDF), 5 % of tokens recomputed identically (ties at 0)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

BLOCK = 16

WORKLOADS = {
    "tiny": dict(index=0, batch=2, lens=(37, 50), n_h=4, n_kv=2, d=64, dtype="f32",
                 num_blocks=16, seed=0, append=True),
    "llama3_8b": dict(index=1, batch=64, lens=("uniform", 512, 4096), n_h=32, n_kv=8, d=128,
                      dtype="bf16", pool_slack=1.10, seed=1, append=True),
    "llama2_70b": dict(index=2, batch=256, lens=("fixed", 2048), n_h=64, n_kv=8, d=128,
                       dtype="bf16", pool_slack=1.0, seed=2, append=True),
    "kvquant_int4": dict(index=3, batch=64, lens=("uniform", 512, 4096), n_h=32, n_kv=8, d=128,
                         dtype="bf16", pool_slack=1.10, seed=3, append=True, int4=True,
                         outliers=4, outlier_scale=10.0),
    "long_shared": dict(index=4, batch=8, lens=("fixed", 32768), n_h=32, n_kv=32, d=128,
                        dtype="bf16", seed=4, append=False, shared_tokens=16384,
                        chunk_first_block=768, chunk_tokens=4096, delta_range=(1, 16384),
                        rope_base=10000.0),
}

BLEND_WORKLOADS = {
    "blend_select": dict(batch=16, ctx=8192, n_kv=8, d=128, dtype="bf16", seed=5, unchanged=0.05,
                         ratio=0.15),
}

# sub-stream ids, one per kind of tensor
(_S_LENS, _S_PERM, _S_K, _S_V, _S_Q, _S_KNEW, _S_VNEW, _S_OUTL, _S_DELTA, _S_SIGMA, _S_KRE, _S_VRE,
 _S_ROWS) = range(13)


def _gen(seed: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + stream * 7919 + 17)
    return g


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def normal(shape, seed: int, stream: int, device, dtype: torch.dtype, scale_channels=None,
           chunk_rows: int = 1 << 16) -> torch.Tensor:
    """N(0,1) in fp32 rounded to `dtype` (round to nearest even).

    scale_channels: optional (channels [n_kv][k], factor) — multiplies the given
    last-axis channels of every kv head (axis 1) by factor before the cast.
    Large tensors are drawn in slabs along the first axis so that the fp32
    temporary stays small."""
    g = _gen(seed, stream, device)
    out = torch.empty(shape, dtype=dtype, device=device)
    n0 = shape[0]
    for s in range(0, n0, chunk_rows):
        e = min(n0, s + chunk_rows)
        x = torch.randn((e - s,) + tuple(shape[1:]), generator=g, device=device, dtype=torch.float32)
        if scale_channels is not None:
            chans, factor = scale_channels
            for h in range(chans.shape[0]):
                x[:, h, ..., chans[h]] *= factor
        out[s:e] = x.to(dtype)
    return out


@dataclass
class Case:
    """One decode step's inputs. Pools are [num_blocks][n_kv][16][d]."""
    name: str
    batch: int
    n_h: int
    n_kv: int
    d: int
    dtype: str                 # "f32" or "bf16" (pool / q / new-token type)
    num_blocks: int
    tables: torch.Tensor       # int32 [B][max_blocks], -1 where unused
    seq_lens: torch.Tensor     # int32 [B], length before the append
    ctx_lens: torch.Tensor     # int32 [B], tokens attended (after the append)
    K: torch.Tensor
    V: torch.Tensor
    q: torch.Tensor            # [B][n_h][d]
    k_new: torch.Tensor        # [B][n_kv][d]
    v_new: torch.Tensor
    scale: float
    append: bool = True
    int4: bool = False
    outlier_channels: torch.Tensor | None = None
    chunk_blocks: torch.Tensor | None = None   # long_shared: physical ids of the chunk, logical order
    chunk_tokens: int = 0
    delta: int = 0
    rope_base: float = 10000.0
    meta: dict = field(default_factory=dict)

    @property
    def max_blocks(self) -> int:
        return int(self.tables.shape[1])

    @property
    def max_ctx(self) -> int:
        return int(self.ctx_lens.max().item()) if self.batch else 0


def softmax_scale(d: int) -> float:
    """1/sqrt(d_h), rounded to fp32 (the value both sides receive)."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32).item())


def _poison_unused(K: torch.Tensor, V: torch.Tensor, tables: torch.Tensor, valid_lens) -> None:
    """NaN in every slot that is not one of the first valid_lens[b] tokens of
    some sequence (unused blocks, the tail of partial blocks, append slots)."""
    nb = K.shape[0]
    valid = torch.zeros((nb, BLOCK), dtype=torch.bool)
    tab = tables.cpu()
    for b, n in enumerate(valid_lens):
        n = int(n)
        full = n // BLOCK
        ids = tab[b, :full]
        valid[ids.long()] = True
        r = n % BLOCK
        if r:
            valid[int(tab[b, full]), :r] = True
    inv = (~valid).to(K.device)[:, None, :, None]
    K.masked_fill_(inv, float("nan"))
    V.masked_fill_(inv, float("nan"))


def make_case(seed: int, batch: int, lens, n_h: int, n_kv: int, d: int, dtype: str = "bf16",
              num_blocks: int | None = None, pool_slack: float = 1.0, device="cpu",
              append: bool | int = True, max_blocks: int | None = None, poison: bool = True,
              outliers: int = 0, outlier_scale: float = 10.0, name: str = "custom") -> Case:
    """A decode step over private (unshared) blocks.

    lens: the per-sequence lengths before the append (list), or
    ("uniform", lo, hi) / ("fixed", n) drawn with the seed.
    append: False, True (one new token per sequence) or a number n of new
    tokens; with n > 1, q is [B][n][n_h][d] and k_new, v_new [B][n][n_kv][d].
    Every sequence owns ceil((len + new tokens) / 16) blocks; physical ids come
    from a seeded permutation of the pool, handed out in logical order."""
    n_new = int(append)
    if isinstance(lens, tuple) and lens and isinstance(lens[0], str):
        if lens[0] == "uniform":
            g = _gen(seed, _S_LENS, "cpu")
            lens_t = torch.randint(lens[1], lens[2] + 1, (batch,), generator=g, dtype=torch.int64)
        else:
            lens_t = torch.full((batch,), int(lens[1]), dtype=torch.int64)
    else:
        lens_t = torch.tensor(list(lens), dtype=torch.int64)
    assert len(lens_t) == batch
    ctx = lens_t + n_new
    need = [(int(c) + BLOCK - 1) // BLOCK for c in ctx]
    total = sum(need)
    if num_blocks is None:
        num_blocks = max(1, int(math.ceil(pool_slack * total)))
    assert num_blocks >= total, "pool too small for the sequences"
    mb = max(need) if need else 1
    mb = max(mb, 1) if max_blocks is None else max_blocks
    perm = torch.randperm(num_blocks, generator=_gen(seed, _S_PERM, "cpu")).to(torch.int32)
    tables = torch.full((batch, mb), -1, dtype=torch.int32)
    off = 0
    for b in range(batch):
        tables[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    tdt = torch_dtype(dtype)
    shape = (num_blocks, n_kv, BLOCK, d)
    outl = None
    sc = None
    if outliers:
        g = _gen(seed, _S_OUTL, "cpu")
        outl = torch.stack([torch.randperm(d, generator=g)[:outliers] for _ in range(n_kv)])
        sc = (outl, outlier_scale)
    K = normal(shape, seed, _S_K, device, tdt, scale_channels=sc)
    V = normal(shape, seed, _S_V, device, tdt)
    if poison:
        _poison_unused(K, V, tables, lens_t.tolist())
    lead = (batch,) if n_new <= 1 else (batch, n_new)
    q = normal(lead + (n_h, d), seed, _S_Q, device, tdt)
    if sc is not None and n_new > 1:
        sc = (sc[0], sc[1])
        k_new = normal(lead + (n_kv, d), seed, _S_KNEW, device, tdt)
        for h in range(n_kv):
            k_new[..., h, sc[0][h]] = (k_new[..., h, sc[0][h]].float() * sc[1]).to(tdt)
    else:
        k_new = normal(lead + (n_kv, d), seed, _S_KNEW, device, tdt, scale_channels=sc)
    v_new = normal(lead + (n_kv, d), seed, _S_VNEW, device, tdt)
    return Case(name=name, batch=batch, n_h=n_h, n_kv=n_kv, d=d, dtype=dtype,
                num_blocks=num_blocks, tables=tables.to(device),
                seq_lens=lens_t.to(torch.int32).to(device), ctx_lens=ctx.to(torch.int32).to(device),
                K=K, V=V, q=q, k_new=k_new, v_new=v_new, scale=softmax_scale(d), append=n_new > 0,
                outlier_channels=outl, meta={"n_new": n_new})


def make_shared_prefix_case(seed: int, batch: int, ctx: int, shared_tokens: int, n_h: int, n_kv: int,
                            d: int, chunk_first_block: int, chunk_tokens: int, delta_range,
                            rope_base: float, dtype: str = "bf16", device="cpu",
                            name: str = "long_shared") -> Case:
    """Sequences whose first shared_tokens tokens map to the same physical
    blocks in every table, the rest private. The reused chunk is the
    chunk_tokens tokens starting at logical block chunk_first_block of the
    shared prefix; its rotation offset is drawn from delta_range."""
    assert shared_tokens % BLOCK == 0 and ctx % BLOCK == 0
    n_shared = shared_tokens // BLOCK
    n_priv = (ctx - shared_tokens) // BLOCK
    num_blocks = n_shared + batch * n_priv
    perm = torch.randperm(num_blocks, generator=_gen(seed, _S_PERM, "cpu")).to(torch.int32)
    mb = n_shared + n_priv
    tables = torch.empty((batch, mb), dtype=torch.int32)
    tables[:, :n_shared] = perm[:n_shared]
    for b in range(batch):
        s = n_shared + b * n_priv
        tables[b, n_shared:] = perm[s:s + n_priv]
    tdt = torch_dtype(dtype)
    shape = (num_blocks, n_kv, BLOCK, d)
    K = normal(shape, seed, _S_K, device, tdt)
    V = normal(shape, seed, _S_V, device, tdt)
    q = normal((batch, n_h, d), seed, _S_Q, device, tdt)
    k_new = normal((batch, n_kv, d), seed, _S_KNEW, device, tdt)
    v_new = normal((batch, n_kv, d), seed, _S_VNEW, device, tdt)
    lo, hi = delta_range
    delta = int(torch.randint(lo, hi + 1, (1,), generator=_gen(seed, _S_DELTA, "cpu")).item())
    chunk_blocks = tables[0, chunk_first_block:chunk_first_block + chunk_tokens // BLOCK].clone()
    lens = torch.full((batch,), ctx, dtype=torch.int32)
    return Case(name=name, batch=batch, n_h=n_h, n_kv=n_kv, d=d, dtype=dtype, num_blocks=num_blocks,
                tables=tables.to(device), seq_lens=lens.to(device), ctx_lens=lens.to(device),
                K=K, V=V, q=q, k_new=k_new, v_new=v_new, scale=softmax_scale(d), append=False,
                chunk_blocks=chunk_blocks.to(device), chunk_tokens=chunk_tokens, delta=delta,
                rope_base=rope_base)


def workload(name: str, device="cpu", poison: bool = True, n_new: int | None = None) -> Case:
    """The named workload at full size. n_new overrides the number of tokens
    appended per sequence (several: a verification step of speculated tokens)."""
    w = WORKLOADS[name]
    if name == "long_shared":
        return make_shared_prefix_case(w["seed"], w["batch"], w["lens"][1], w["shared_tokens"], w["n_h"],
                                       w["n_kv"], w["d"], w["chunk_first_block"], w["chunk_tokens"],
                                       w["delta_range"], w["rope_base"], w["dtype"], device, name)
    c = make_case(w["seed"], w["batch"], w["lens"], w["n_h"], w["n_kv"], w["d"], w["dtype"],
                  num_blocks=w.get("num_blocks"), pool_slack=w.get("pool_slack", 1.0), device=device,
                  append=w["append"] if n_new is None else n_new, poison=poison, outliers=w.get("outliers", 0),
                  outlier_scale=w.get("outlier_scale", 10.0), name=name)
    c.int4 = bool(w.get("int4", False))
    return c


@dataclass
class BlendCase:
    """Selection inputs: a pool holding each request's reused tokens and the
    recomputed K/V of a set of rows (row i: token row_pos[i] of request
    row_seq[i]); rows of request s are rows seg_offsets[s] .. seg_offsets[s+1]."""
    name: str
    batch: int
    n_kv: int
    d: int
    dtype: str
    num_blocks: int
    tables: torch.Tensor       # int32 [B][max_blocks]
    K: torch.Tensor
    V: torch.Tensor
    row_seq: torch.Tensor      # int32 [rows]
    row_pos: torch.Tensor      # int32 [rows]
    k_re: torch.Tensor         # [rows][n_kv][d]
    v_re: torch.Tensor
    seg_offsets: torch.Tensor  # int32 [B + 1]
    sigma2: torch.Tensor       # fp32 [rows], the drawn noise variance per row

    @property
    def n_rows(self) -> int:
        return int(self.row_seq.numel())


def make_blend_case(seed: int, batch: int, ctx: int, n_kv: int, d: int, dtype: str = "bf16",
                    unchanged: float = 0.05, rows_per_seq: int | None = None, device="cpu",
                    name: str = "custom") -> BlendCase:
    """Every request owns ctx cached tokens in private blocks (seeded
    permutation of the pool). rows_per_seq None: a row for every cached token
    in position order (the wide first-layer candidate set); else that many
    seeded distinct positions per request, ascending (a narrowed set).
    Recomputed row = cached row + sigma * N(0, 1) per element, cast to the
    pool type, with sigma^2 ~ U(0, 1) per row and sigma = 0 for a seeded
    `unchanged` fraction of rows."""
    base = make_case(seed, batch, [ctx] * batch, n_kv, n_kv, d, dtype, append=False, poison=False,
                     device=device, name=name)
    tables = base.tables.to("cpu")
    if rows_per_seq is None:
        pos = torch.arange(ctx, dtype=torch.int64).repeat(batch)
        per = [ctx] * batch
    else:
        g = _gen(seed, _S_ROWS, "cpu")
        pos = torch.cat([torch.randperm(ctx, generator=g)[:rows_per_seq].sort().values for _ in range(batch)])
        per = [min(rows_per_seq, ctx)] * batch
    seq = torch.cat([torch.full((n,), b, dtype=torch.int64) for b, n in enumerate(per)]) if batch else \
        torch.zeros(0, dtype=torch.int64)
    n_rows = int(seq.numel())
    g = _gen(seed, _S_SIGMA, "cpu")
    sigma2 = torch.rand(n_rows, generator=g)
    sigma2[torch.rand(n_rows, generator=g) < unchanged] = 0.0
    blk = tables[seq, pos // BLOCK].to(torch.int64).to(device)
    slot = (pos % BLOCK).to(device)
    tdt = torch_dtype(dtype)
    sig = sigma2.sqrt().to(device)[:, None, None]
    k_re = torch.empty((n_rows, n_kv, d), dtype=tdt, device=device)
    v_re = torch.empty_like(k_re)
    step = 1 << 15
    gk, gv = _gen(seed, _S_KRE, device), _gen(seed, _S_VRE, device)
    for s in range(0, n_rows, step):
        e = min(n_rows, s + step)
        nk = torch.randn((e - s, n_kv, d), generator=gk, device=device)
        nv = torch.randn((e - s, n_kv, d), generator=gv, device=device)
        k_re[s:e] = (base.K[blk[s:e], :, slot[s:e], :].float() + sig[s:e] * nk).to(tdt)
        v_re[s:e] = (base.V[blk[s:e], :, slot[s:e], :].float() + sig[s:e] * nv).to(tdt)
    offs = torch.zeros(batch + 1, dtype=torch.int32)
    if batch:
        offs[1:] = torch.tensor(per, dtype=torch.int64).cumsum(0).to(torch.int32)
    return BlendCase(name=name, batch=batch, n_kv=n_kv, d=d, dtype=dtype, num_blocks=base.num_blocks,
                     tables=base.tables, K=base.K, V=base.V, row_seq=seq.to(torch.int32).to(device),
                     row_pos=pos.to(torch.int32).to(device), k_re=k_re, v_re=v_re,
                     seg_offsets=offs.to(device), sigma2=sigma2)


def blend_workload(name: str, device="cpu", rows_per_seq: int | None = None) -> BlendCase:
    w = BLEND_WORKLOADS[name]
    return make_blend_case(w["seed"], w["batch"], w["ctx"], w["n_kv"], w["d"], w["dtype"], w["unchanged"],
                           rows_per_seq, device, name)


def to_host_bits(t: torch.Tensor):
    """Host numpy copy: f32 stays f32, bf16 becomes its uint16 bit pattern."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
