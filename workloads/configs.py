"""The five synthetic batches the hot path is checked and measured on.

Each generator returns a `Workload`: the structure of one step of a paged KV
cache (context lengths, per-sequence block tables into a shared pool, which
pool slots hold valid data before the step, the tokens this step appends and
the copy-on-write block pairs it needs) plus the recipe for every tensor's
values.  Lengths and placements come from NumPy's PCG64 seeded with the
config's seed; tensor values come from the counter-based generator in gen.py.

Structure follows the workloads the pages describe:
  * blocks of 16 tokens placed anywhere in one shared pool, through a
    per-sequence table [P1 "Efficient Memory Management for Large Language
    Model Serving with PagedAttention", sec. 5, Fig. 7 and Fig. 8];
  * prompt blocks shared by parallel samples, with a copy-on-write of the
    partially filled last shared block at the first divergent write
    [P1 sec. 6, Fig. 9; P2 "SOSP 2023論文解説: vLLM — PagedAttentionによる
    KVキャッシュメモリ管理の革新", pseudocode section];
  * chunked prefill interleaved with decodes in one batch [P3 "연속 배치 처리
    아키텍처", Chunked prefill];
  * long-tailed request lengths (a lognormal stands in for the chat-log
    length histogram of P1 sec. 7, Fig. 12).

Tensor stream ids: 1 = K pool, 2 = V pool, 3 = q, 4 = new K rows, 5 = new V rows,
6 = the per-(head, dim) signs of marked values.
Pool slots that hold no valid data before the step are NaN.

Value recipes (a Workload's `values`, `k_scale`, `v_mark`):
  * "exact" (default for fp16): every value is on the 1/256 grid (exact in fp16);
  * "full" (default for fp32 decode batches): full-mantissa fp32 values, not
    representable in fp16, so an fp32 path that rounds through fp16 is seen;
  * k_scale (a power of two) multiplies every key, exactly: small keys make
    the scores nearly equal, so every token carries a similar weight;
  * v_mark = A > 0 marks the values by block: the value of head h, dim c of a
    token in logical block b of its sequence is A * (-1)^b * r(h, c) plus the
    usual noise (computed in fp32, rounded once to the dtype), r = +-1 per
    (head, dim); the one token a decode sequence appends this step carries
    B * A instead (B = block size), so on its own it weighs like a whole block
    (tokens of a multi-token append, a prefill chunk, carry A).  Neighbouring blocks
    pull every output element in opposite directions, so the output stays
    small while leaving out any one block (or the appended token) moves it by
    about A * B times that block's weight: a test on such inputs sees a
    dropped, repeated or misplaced block.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from .gen import normal_array, normal_values, normal_values_torch, values_at_torch

STREAM_K, STREAM_V, STREAM_Q, STREAM_KNEW, STREAM_VNEW, STREAM_MARK = 1, 2, 3, 4, 5, 6

CONFIG_NAMES = {
    1: "tiny_decode_f32",
    2: "13b_decode_b64",
    3: "parallel_sampling_cow",
    4: "chunked_prefill_mixed",
    5: "large_batch_decode_write",
}


@dataclass
class Workload:
    name: str
    seed: int
    dtype: str                      # "f32" | "f16"
    num_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    context_lens: np.ndarray        # int32 [S]: tokens per sequence after this step's writes
    query_lens: np.ndarray          # int32 [S]: queries per sequence for attention (>= 1)
    write_lens: np.ndarray          # int32 [S]: tokens appended this step (0 = none)
    block_tables: np.ndarray        # int32 [S][max_blocks], -1 beyond the used entries
    filled_before: np.ndarray       # int32 [NB]: leading slots of each block valid before the step
    copy_pairs: Optional[np.ndarray] = None   # int32 [n][2] = (src, dst), or None
    q_scale: float = 1.0            # power of two applied to q
    extra: dict = field(default_factory=dict)
    values: str = "exact"           # "exact" (1/256 grid) | "full" (full-mantissa fp32)
    k_scale: float = 1.0            # power of two applied to every key
    v_mark: float = 0.0             # > 0: block-alternating value marks of this amplitude

    def __post_init__(self):
        if self.values not in ("exact", "full"):
            raise ValueError(f"unknown value recipe {self.values!r}")
        if self.values == "full" and self.dtype != "f32":
            raise ValueError("full-mantissa values are for fp32 batches")

    # ----- derived sizes -------------------------------------------------
    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_queries(self) -> int:
        return int(self.query_lens.sum())

    @property
    def num_writes(self) -> int:
        return int(self.write_lens.sum())

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def np_dtype(self):
        return np.float32 if self.dtype == "f32" else np.float16

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max())

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max())

    def q_start_loc(self) -> Optional[np.ndarray]:
        """int32 [S+1] prefix sums of query_lens, or None when every sequence has one query."""
        if np.all(self.query_lens == 1):
            return None
        return np.concatenate([[0], np.cumsum(self.query_lens)]).astype(np.int32)

    def write_start_loc(self) -> Optional[np.ndarray]:
        if np.all(self.write_lens == 1):
            return None
        return np.concatenate([[0], np.cumsum(self.write_lens)]).astype(np.int32)

    def kv_bytes_read(self) -> int:
        """K/V bytes an attention pass must read: every valid row of every context once."""
        return int(2 * self.context_lens.astype(np.int64).sum() * self.num_heads * self.head_dim
                   * self.elt_bytes)

    def unique_blocks_read(self) -> int:
        used = set()
        B = self.block_size
        for s in range(self.num_seqs):
            nb = -(-int(self.context_lens[s]) // B)
            used.update(int(x) for x in self.block_tables[s, :nb])
        return len(used)

    def shares_blocks(self) -> bool:
        """Whether any physical block is read by more than one sequence."""
        B = self.block_size
        total = sum(-(-int(L) // B) for L in self.context_lens)
        return self.unique_blocks_read() < total

    # ----- tensors -------------------------------------------------------
    def pool_shape(self):
        return (self.num_blocks, self.block_size, self.num_heads, self.head_dim)

    def _valid_mask(self) -> np.ndarray:
        slots = np.arange(self.block_size, dtype=np.int32)
        return slots[None, :] < self.filled_before[:, None]          # [NB][B]

    # ----- value marks ---------------------------------------------------
    def block_signs(self) -> np.ndarray:
        """int8 [NB]: (-1)^b for a block at logical index b of the first sequence holding it
        (+1 for blocks no sequence holds)."""
        sign = np.zeros(self.num_blocks, np.int8)
        B = self.block_size
        for s in range(self.num_seqs):
            nb = -(-int(self.context_lens[s]) // B)
            row = self.block_tables[s, :nb]
            fresh = sign[row] == 0
            sign[row[fresh]] = np.where(np.arange(nb)[fresh] % 2 == 0, 1, -1)
        if self.copy_pairs is not None:
            for src, dst in self.copy_pairs:
                if sign[dst] == 0:
                    sign[dst] = sign[src]
        sign[sign == 0] = 1
        return sign

    def write_signs(self) -> np.ndarray:
        """float32 [num_writes]: the mark factor of each appended token, (-1)^b with b its
        logical block, times the block size when it is its sequence's only appended token."""
        out = np.empty(self.num_writes, np.float32)
        r = 0
        for s in range(self.num_seqs):
            L, n = int(self.context_lens[s]), int(self.write_lens[s])
            for i in range(n):
                sign = 1.0 if ((L - n + i) // self.block_size) % 2 == 0 else -1.0
                out[r] = sign * (self.block_size if n == 1 else 1)
                r += 1
        return out

    def head_dim_signs(self) -> np.ndarray:
        """float32 [H][d]: r(h, c) = +-1."""
        H, D = self.num_heads, self.head_dim
        x = normal_values(self.seed, STREAM_MARK, np.arange(H * D, dtype=np.int64), np.float64)
        return np.where(x >= 0, 1.0, -1.0).astype(np.float32).reshape(H, D)

    def host_block_rows(self, blocks, heads=None) -> dict:
        """Pool contents before the step of the given physical blocks, for the given heads only
        (all when None): {"k_pool", "v_pool"} arrays [n][B][len(heads)][d] of the dtype, NaN in
        unfilled slots; the same values host_tensors() / device_tensors() hold there."""
        import torch

        blocks = np.asarray(blocks, np.int64)
        H, D, B = self.num_heads, self.head_dim, self.block_size
        heads = np.arange(H) if heads is None else np.asarray(heads, np.int64)
        full = self.values == "full"
        idx = (((blocks[:, None, None, None] * B + np.arange(B)[None, :, None, None]) * H
                + heads[None, None, :, None]) * D + np.arange(D)[None, None, None, :])
        it = torch.from_numpy(np.ascontiguousarray(idx))
        dt = self.np_dtype
        k = values_at_torch(self.seed, STREAM_K, it, full).numpy().astype(dt)
        k = k * dt(self.k_scale)
        if self.v_mark:
            v32 = values_at_torch(self.seed, STREAM_V, it, full).numpy().astype(np.float32)
            mark = np.float32(self.v_mark) * self.block_signs()[blocks].astype(np.float32)
            r = self.head_dim_signs()[heads]
            v = (v32 + mark[:, None, None, None] * r[None, None]).astype(dt)
        else:
            v = values_at_torch(self.seed, STREAM_V, it, full).numpy().astype(dt)
        invalid = np.arange(B)[None, :] >= self.filled_before[blocks][:, None]
        k[invalid] = np.nan
        v[invalid] = np.nan
        return {"k_pool": k, "v_pool": v}

    def host_new_rows(self, heads=None) -> dict:
        """This step's appended rows {"k_new", "v_new"} [num_writes][len(heads)][d] for the given
        heads only (all when None), as host_tensors() holds them."""
        import torch

        H, D = self.num_heads, self.head_dim
        heads = np.arange(H) if heads is None else np.asarray(heads, np.int64)
        full = self.values == "full"
        dt = self.np_dtype
        idx = ((np.arange(self.num_writes)[:, None, None] * H + heads[None, :, None]) * D
               + np.arange(D)[None, None, :])
        it = torch.from_numpy(np.ascontiguousarray(idx))
        k = values_at_torch(self.seed, STREAM_KNEW, it, full).numpy().astype(dt) * dt(self.k_scale)
        if self.v_mark:
            v32 = values_at_torch(self.seed, STREAM_VNEW, it, full).numpy().astype(np.float32)
            mark = np.float32(self.v_mark) * self.write_signs()
            v = (v32 + mark[:, None, None] * self.head_dim_signs()[heads][None]).astype(dt)
        else:
            v = values_at_torch(self.seed, STREAM_VNEW, it, full).numpy().astype(dt)
        return {"k_new": k.astype(dt), "v_new": v}

    def host_tensors(self) -> dict:
        """All inputs as NumPy arrays (small workloads only)."""
        dt = self.np_dtype
        H, D = self.num_heads, self.head_dim
        full = self.values == "full"
        k_pool = normal_array(self.seed, STREAM_K, self.pool_shape(), dt, full=full)
        k_pool *= dt(self.k_scale)
        if self.v_mark:
            v32 = normal_array(self.seed, STREAM_V, self.pool_shape(), np.float32, full=full)
            mark = np.float32(self.v_mark) * self.block_signs().astype(np.float32)
            v_pool = (v32 + mark[:, None, None, None] * self.head_dim_signs()[None, None]).astype(dt)
        else:
            v_pool = normal_array(self.seed, STREAM_V, self.pool_shape(), dt, full=full)
        invalid = ~self._valid_mask()
        k_pool[invalid] = np.nan
        v_pool[invalid] = np.nan
        q = normal_array(self.seed, STREAM_Q, (self.num_queries, H, D), dt, full=full)
        q = q * dt(self.q_scale)
        out = dict(k_pool=k_pool, v_pool=v_pool, q=q.astype(dt))
        if self.num_writes:
            kn = normal_array(self.seed, STREAM_KNEW, (self.num_writes, H, D), dt, full=full)
            out["k_new"] = (kn * dt(self.k_scale)).astype(dt)
            if self.v_mark:
                v32 = normal_array(self.seed, STREAM_VNEW, (self.num_writes, H, D), np.float32,
                                   full=full)
                mark = np.float32(self.v_mark) * self.write_signs()
                out["v_new"] = (v32 + mark[:, None, None] * self.head_dim_signs()[None]).astype(dt)
            else:
                out["v_new"] = normal_array(self.seed, STREAM_VNEW, (self.num_writes, H, D), dt,
                                            full=full)
        out.update(self._index_arrays())
        return out

    def _index_arrays(self) -> dict:
        out = dict(
            block_tables=np.ascontiguousarray(self.block_tables, dtype=np.int32),
            context_lens=np.ascontiguousarray(self.context_lens, dtype=np.int32),
            q_start_loc=self.q_start_loc(),
            write_start_loc=self.write_start_loc(),
        )
        if self.copy_pairs is not None:
            out["copy_pairs"] = np.ascontiguousarray(self.copy_pairs, dtype=np.int32)
        return out

    def device_tensors(self, device="cuda") -> dict:
        """All inputs as torch tensors on `device`, generated in place there."""
        import torch

        tdt = torch.float32 if self.dtype == "f32" else torch.float16
        H, D = self.num_heads, self.head_dim
        full = self.values == "full"
        hd_sign = (torch.from_numpy(self.head_dim_signs()).to(device) if self.v_mark else None)

        def marked(shape, stream, signs, amp):
            """amp * sign * r(h, c) + noise, in fp32, rounded once to the dtype."""
            t32 = torch.empty(shape, dtype=torch.float32, device=device)
            normal_values_torch(self.seed, stream, t32, full=full)
            sg = torch.from_numpy(signs.astype(np.float32)).to(device) * float(amp)
            view = t32.view(shape[0], -1, H, D)
            for a in range(0, shape[0], 4096):   # bounded temporaries on large pools
                view[a:a + 4096] += sg[a:a + 4096, None, None, None] * hd_sign[None, None]
            return t32.to(tdt)

        out = {}
        mask = torch.from_numpy(~self._valid_mask()).to(device)
        for name, stream in (("k_pool", STREAM_K), ("v_pool", STREAM_V)):
            if name == "v_pool" and self.v_mark:
                t = marked(self.pool_shape(), stream, self.block_signs(), self.v_mark)
            else:
                t = torch.empty(self.pool_shape(), dtype=tdt, device=device)
                normal_values_torch(self.seed, stream, t, full=full)
                if name == "k_pool" and self.k_scale != 1.0:
                    t.mul_(self.k_scale)
            t.view(self.num_blocks, self.block_size, H * D)[mask] = float("nan")
            out[name] = t
        q = torch.empty((self.num_queries, H, D), dtype=tdt, device=device)
        normal_values_torch(self.seed, STREAM_Q, q, full=full)
        out["q"] = q * self.q_scale
        if self.num_writes:
            for name, stream in (("k_new", STREAM_KNEW), ("v_new", STREAM_VNEW)):
                if name == "v_new" and self.v_mark:
                    t = marked((self.num_writes, H, D), stream, self.write_signs(),
                               self.v_mark)
                else:
                    t = torch.empty((self.num_writes, H, D), dtype=tdt, device=device)
                    normal_values_torch(self.seed, stream, t, full=full)
                    if name == "k_new" and self.k_scale != 1.0:
                        t.mul_(self.k_scale)
                out[name] = t
        for k, v in self._index_arrays().items():
            out[k] = None if v is None else torch.from_numpy(v).to(device)
        return out


# ---------------------------------------------------------------------------
# structure helpers
# ---------------------------------------------------------------------------

def _cdiv(a, b):
    return -(-a // b)


def _tables_from_permutation(rng, lens, block_size, num_blocks, pad=1):
    """Give each sequence ceil(len/B) blocks taken in order from a random permutation."""
    need = [_cdiv(int(L), block_size) for L in lens]
    if sum(need) > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {sum(need)}")
    perm = rng.permutation(num_blocks).astype(np.int32)
    width = max(need) + pad
    bt = np.full((len(lens), width), -1, dtype=np.int32)
    pos = 0
    for s, n in enumerate(need):
        bt[s, :n] = perm[pos:pos + n]
        pos += n
    return bt


def _filled_from_tables(bt, lens_before, block_size, num_blocks):
    filled = np.zeros(num_blocks, dtype=np.int32)
    for s, L in enumerate(lens_before):
        L = int(L)
        for b in range(_cdiv(L, block_size)):
            filled[bt[s, b]] = max(filled[bt[s, b]], min(block_size, L - b * block_size))
    return filled


def _decode_workload(name, seed, dtype, H, D, B, lens, num_blocks, write_one=False, q_scale=1.0,
                     rng=None, **recipe):
    rng = rng if rng is not None else np.random.default_rng(seed)
    # fp32 batches take full-mantissa values unless told otherwise (see the module docstring)
    recipe.setdefault("values", "full" if dtype == "f32" else "exact")
    lens = np.asarray(lens, dtype=np.int32)
    bt = _tables_from_permutation(rng, lens, B, num_blocks)
    S = len(lens)
    write_lens = np.ones(S, np.int32) if write_one else np.zeros(S, np.int32)
    filled = _filled_from_tables(bt, lens - write_lens, B, num_blocks)
    return Workload(name=name, seed=seed, dtype=dtype, num_heads=H, head_dim=D, block_size=B,
                    num_blocks=num_blocks, context_lens=lens, query_lens=np.ones(S, np.int32),
                    write_lens=write_lens, block_tables=bt, filled_before=filled, q_scale=q_scale,
                    **recipe)


def _lognormal_lens(rng, n, median, sigma, lo, hi):
    x = np.exp(rng.normal(np.log(median), sigma, size=n))
    return np.clip(np.rint(x), lo, hi).astype(np.int32)


# ---------------------------------------------------------------------------
# the five configurations
# ---------------------------------------------------------------------------

def config1(seed=1, values="full", **_):
    """Tiny decode: 4 seqs, 2 heads, d=64, B=16, fp32, lengths U{1..100}, pool of 64 blocks."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 101, size=4)
    return _decode_workload(CONFIG_NAMES[1], seed, "f32", 2, 64, 16, lens, 64, rng=rng,
                            values=values)


def _recipe(kw):
    """The value-recipe arguments among a config's keyword arguments."""
    return {k: kw[k] for k in ("values", "k_scale", "v_mark") if k in kw}


def config2(seed=2, num_seqs=64, num_heads=40, median=512, max_len=2048, block_size=16,
            q_scale=1.0, **kw):
    """13B-shaped single-layer decode: lognormal lengths (sigma 1), pool 1.25x the need."""
    rng = np.random.default_rng(seed)
    lens = _lognormal_lens(rng, num_seqs, median, 1.0, 1, max_len)
    need = int(sum(_cdiv(int(L), block_size) for L in lens))
    nb = _cdiv(5 * need, 4)
    return _decode_workload(CONFIG_NAMES[2], seed, "f16", num_heads, 128, block_size, lens, nb,
                            q_scale=q_scale, rng=rng, **_recipe(kw))


def config3(seed=3, num_prompts=16, prompt_len=1000, samples=6, max_gen=300, num_heads=40,
            block_size=16, **kw):
    """Parallel sampling: samples share a prompt's blocks; the partial last prompt block is
    copied on the first divergent write by every sharer but the last (refcount reaches 1)."""
    rng = np.random.default_rng(seed)
    B = block_size
    nprompt_blocks = _cdiv(prompt_len, B)
    partial = prompt_len % B != 0
    gens = rng.integers(1, max_gen + 1, size=(num_prompts, samples)).astype(np.int32)
    # blocks each sample needs beyond the shared prompt blocks
    free_in_last = (B - prompt_len % B) % B
    extra_blocks = [[_cdiv(max(0, int(g) - free_in_last), B) for g in row] for row in gens]
    ncopies = (samples - 1) if partial else 0
    need = num_prompts * (nprompt_blocks + ncopies) + int(sum(map(sum, extra_blocks)))
    nb = _cdiv(5 * need, 4)
    perm = iter(rng.permutation(nb).astype(np.int32).tolist())

    S = num_prompts * samples
    lens = (prompt_len + gens.reshape(-1)).astype(np.int32)
    width = max(_cdiv(int(L), B) for L in lens) + 1
    bt = np.full((S, width), -1, np.int32)
    filled = np.zeros(nb, np.int32)
    pairs = []
    for p in range(num_prompts):
        shared = [next(perm) for _ in range(nprompt_blocks)]
        for i, blk in enumerate(shared):
            filled[blk] = min(B, prompt_len - i * B)
        for k in range(samples):
            s = p * samples + k
            row = list(shared)
            if partial and k < samples - 1:
                dst = next(perm)              # NaN until the copy brings the prompt's partial block
                pairs.append((shared[-1], dst))
                row[-1] = dst
            row += [next(perm) for _ in range(extra_blocks[p][k])]
            bt[s, :len(row)] = row
    return Workload(name=CONFIG_NAMES[3], seed=seed, dtype="f16", num_heads=num_heads,
                    head_dim=128, block_size=B, num_blocks=nb, context_lens=lens,
                    query_lens=np.ones(S, np.int32), write_lens=gens.reshape(-1).copy(),
                    block_tables=bt, filled_before=filled,
                    copy_pairs=np.asarray(pairs, np.int32).reshape(-1, 2),
                    extra=dict(prompt_len=prompt_len, samples=samples, num_prompts=num_prompts),
                    **_recipe(kw))


def config4(seed=4, num_chunks=8, chunk=512, max_prior=2048, num_decodes=56, max_decode_len=2048,
            num_heads=32, block_size=16, **kw):
    """Chunked prefill: chunk queries attend causally to prior paged tokens plus themselves,
    mixed in one batch with single-token decodes (order shuffled)."""
    rng = np.random.default_rng(seed)
    prior = rng.integers(0, max_prior + 1, size=num_chunks)
    dec = rng.integers(1, max_decode_len + 1, size=num_decodes)
    lens = np.concatenate([prior + chunk, dec]).astype(np.int32)
    qlens = np.concatenate([np.full(num_chunks, chunk), np.ones(num_decodes)]).astype(np.int32)
    order = rng.permutation(len(lens))
    lens, qlens = lens[order], qlens[order]
    need = int(sum(_cdiv(int(L), block_size) for L in lens))
    nb = _cdiv(5 * need, 4)
    bt = _tables_from_permutation(rng, lens, block_size, nb)
    filled = _filled_from_tables(bt, lens - qlens, block_size, nb)
    return Workload(name=CONFIG_NAMES[4], seed=seed, dtype="f16", num_heads=num_heads,
                    head_dim=128, block_size=block_size, num_blocks=nb, context_lens=lens,
                    query_lens=qlens, write_lens=qlens.copy(), block_tables=bt,
                    filled_before=filled, **_recipe(kw))


def config5(seed=5, num_seqs=256, num_heads=40, min_len=1024, max_len=4096, num_blocks=47104,
            block_size=16, **kw):
    """Large-batch decode with a one-token KV append per sequence, pool of 47,104 blocks."""
    rng = np.random.default_rng(seed)
    lens0 = rng.integers(min_len, max_len + 1, size=num_seqs)
    return _decode_workload(CONFIG_NAMES[5], seed, "f16", num_heads, 128, block_size, lens0 + 1,
                            num_blocks, write_one=True, rng=rng, **_recipe(kw))


def make_custom_decode(seed, dtype, num_heads, head_dim, block_size, lens, num_blocks=None,
                       write_one=False, q_scale=1.0, name="custom_decode", **recipe):
    """One query per sequence with the given context lengths; tables from a random permutation
    of a pool 1.25x the blocks needed (or num_blocks).  recipe: values / k_scale / v_mark."""
    lens = np.asarray(lens, dtype=np.int32)
    need = int(sum(_cdiv(int(L), block_size) for L in lens))
    nb = num_blocks if num_blocks is not None else max(need + 2, _cdiv(5 * need, 4))
    return _decode_workload(name, seed, dtype, num_heads, head_dim, block_size, lens, nb,
                            write_one=write_one, q_scale=q_scale, **recipe)


def make_custom_mixed(seed, num_heads, block_size, chunks, decode_lens, name="custom_mixed",
                      q_scale=1.0, head_dim=128, **recipe):
    """Chunks (prior tokens, new tokens) attending causally, plus single-token decodes, in one
    batch (order shuffled); every new token is also appended this step."""
    rng = np.random.default_rng(seed)
    lens = [p + n for p, n in chunks] + list(decode_lens)
    qlens = [n for _, n in chunks] + [1] * len(decode_lens)
    order = rng.permutation(len(lens))
    lens = np.asarray(lens, np.int32)[order]
    qlens = np.asarray(qlens, np.int32)[order]
    need = int(sum(_cdiv(int(L), block_size) for L in lens))
    nb = max(need + 2, _cdiv(5 * need, 4))
    bt = _tables_from_permutation(rng, lens, block_size, nb)
    filled = _filled_from_tables(bt, lens - qlens, block_size, nb)
    return Workload(name=name, seed=seed, dtype="f16", num_heads=num_heads, head_dim=head_dim,
                    block_size=block_size, num_blocks=nb, context_lens=lens, query_lens=qlens,
                    write_lens=qlens.copy(), block_tables=bt, filled_before=filled,
                    q_scale=q_scale, **recipe)


_MAKERS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def make_config(index: int, seed: Optional[int] = None, **kw) -> Workload:
    """Full-size configuration `index` (1..5); the default seed is the index."""
    return _MAKERS[index](seed=index if seed is None else seed, **kw)


# Reduced variants: same structure, sizes the fp64 oracle finishes in seconds while still
# spanning several context partitions and a ragged last block.
_SMALL = {
    1: dict(),
    2: dict(num_seqs=12, num_heads=4, median=400, max_len=2048),
    3: dict(num_prompts=2, samples=3, prompt_len=1000, max_gen=300, num_heads=4),
    4: dict(num_chunks=2, chunk=96, max_prior=700, num_decodes=5, max_decode_len=1500,
            num_heads=4),
    5: dict(num_seqs=6, num_heads=4, min_len=1024, max_len=4096, num_blocks=6 * 260),
}


def make_small(index: int, seed: Optional[int] = None, **kw) -> Workload:
    args = dict(_SMALL[index])
    args.update(kw)
    return make_config(index, seed, **args)
