"""Seeded synthetic inputs for causal attention over a 16-token-block paged KV cache.

This module draws request lengths, physical block placements and N(0,1) values,
rounds them to the storage dtype and lays them out in the cache format
``[num_blocks][16][num_kv_heads][head_dim]``.  It holds none of the attention
arithmetic: the HIP kernels and the CPU oracle both consume what it returns, and
neither is imported here.

Sources (the four web pages on paged attention, cited by page and section):
  P1  "Prefill 和 Decode 不是两个步骤..." (lshu.cn/news/11576)
  P3  prefill/decode article under the page titled "企业官网建设流程全解析"
      (hotelren.com/news/6181127)
  P4  "11. 分块预填充与统一调度" (niuwancheng.cn, llm-inference/11-chunked-prefill)

Readings taken where the pages are silent:
  * a request's ``seq_len`` counts its keys after this step's append (P3 §3.1:
    the new token's K/V are appended first, then attention runs over all keys);
  * every query token of the step also appends its K/V (P4 "把长输入切成块":
    a chunk reads the earlier KV and then writes its own);
  * lengths "uniform in [a, b]" are integers with both ends included; "log-uniform"
    is ``round(exp(U(ln a, ln b)))`` clipped to [a, b];
  * the block pool is shuffled and consecutive slices of it are handed to the
    requests in order, so physical blocks interleave across requests;
  * slots not holding a live token are poisoned (K = +-3e38, V = NaN) and
    block-table padding is -1, so a kernel that reads outside the visible range
    produces non-finite output;
  * 8-bit caches (P2 §4.3, §5.4: INT8 KV, calibrated per channel): activations stay
    bf16; the cached context is drawn directly as int8 codes (N(0,1) * 32 rounded,
    clipped to +-127: about a quarter of the code range, as N(0,1) data under an
    absmax/127 calibration would give) with poison code -128 in unused slots, and
    each (KV head, channel) gets a scale (4/127) * U(0.75, 1.25) for K and for V.
    The step's new tokens are bf16 values that the append itself quantises.
Draw order per workload: lengths -> block permutation -> Q -> K -> V
(-> int8 context codes of K, then of V -> K scales -> V scales).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

BLOCK_SIZE = 16
K_POISON = 3.0e38
I8_POISON = -128
DTYPES = ("f32", "bf16")
CACHE_DTYPES = ("f32", "bf16", "i8")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def esize(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


def np_storage_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32) if dtype == "f32" else f32_to_bf16_bits(x)


_CHUNK = 1 << 24


def normal_storage(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) float32 draws in storage dtype.  Drawn in chunks (the stream is the same as one
    draw of the whole array) so that bf16 rounding never touches full-size temporaries."""
    n = int(np.prod(shape))
    if dtype == "f32":
        return rng.standard_normal(n, dtype=np.float32).reshape(shape)
    out = np.empty(n, dtype=np.uint16)
    for i in range(0, n, _CHUNK):
        m = min(_CHUNK, n - i)
        out[i:i + m] = f32_to_bf16_bits(rng.standard_normal(m, dtype=np.float32))
    return out.reshape(shape)


def int8_codes(rng: np.random.Generator, shape) -> np.ndarray:
    """Synthetic int8 cache content: N(0,1) * 32 rounded to integers, clipped to [-127, 127]
    (drawn in chunks, like normal_storage)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.int8)
    for i in range(0, n, _CHUNK):
        m = min(_CHUNK, n - i)
        out[i:i + m] = np.clip(np.rint(rng.standard_normal(m, dtype=np.float32) * 32.0), -127, 127)
    return out.reshape(shape)


def channel_scales(rng: np.random.Generator, num_kv_heads: int, head_dim: int) -> np.ndarray:
    """One fp32 scale per (KV head, channel): (4/127) * U(0.75, 1.25)."""
    return (np.float32(4.0 / 127.0) * rng.uniform(0.75, 1.25, (num_kv_heads, head_dim))).astype(np.float32)


def to_float(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> float32 view of the values it holds."""
    return np.asarray(x, dtype=np.float32) if dtype == "f32" else bf16_bits_to_f32(x)


def poison_cache(shape, dtype: str, rng_sign: Optional[np.random.Generator] = None):
    """Fresh K and V caches filled with poison: K = +-3e38 (sign alternating along d), V = NaN."""
    d = shape[-1]
    sign = np.where(np.arange(d) % 2 == 0, 1.0, -1.0).astype(np.float32)
    krow = (sign * np.float32(K_POISON)).astype(np.float32)
    kc = np.empty(shape, dtype=np_storage_dtype(dtype))
    vc = np.empty(shape, dtype=np_storage_dtype(dtype))
    if dtype == "f32":
        kc[...] = krow
        vc[...] = np.float32(np.nan)
    else:
        kc[...] = f32_to_bf16_bits(krow)
        vc[...] = np.uint16(0x7FC0)
    return kc, vc


@dataclass
class Step:
    """One call of the hot path: append the step's K/V, then attend.

    Arrays are host numpy in storage dtype (float32, or uint16 bf16 bit patterns).
    """
    q: np.ndarray                 # [T, Hq, d]
    k_new: np.ndarray             # [T, Hkv, d]   K of the step's tokens
    v_new: np.ndarray             # [T, Hkv, d]
    slot_mapping: np.ndarray      # [T] int32, physical slot = block*16 + offset
    seq_lens: np.ndarray          # [B] int32, keys visible after the append
    query_start_loc: np.ndarray   # [B+1] int32
    block_tables: np.ndarray      # [B, MB] int32, padding = -1

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.query_start_loc).astype(np.int64)


@dataclass
class Workload:
    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    scale: float
    k_cache0: np.ndarray          # [NB, 16, Hkv, d] cache contents before the first step
    v_cache0: np.ndarray
    steps: List[Step] = field(default_factory=list)
    seed: int = 0
    description: str = ""
    kv_dtype: str = ""            # cache element type when it differs from dtype ("i8")
    k_scale: Optional[np.ndarray] = None   # [Hkv, d] float32, int8 caches only
    v_scale: Optional[np.ndarray] = None

    @property
    def cache_dtype(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def esz(self) -> int:
        """Bytes per cache element."""
        return 1 if self.cache_dtype == "i8" else esize(self.dtype)


def _alloc_blocks(rng, seq_lens: Sequence[int], num_blocks: int, max_blocks: int, shuffle: bool, pad: int = -1):
    need = [(int(s) + BLOCK_SIZE - 1) // BLOCK_SIZE for s in seq_lens]
    if sum(need) > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks is too small for {sum(need)}")
    if max(need) > max_blocks:
        raise ValueError("max_blocks too small")
    perm = rng.permutation(num_blocks).astype(np.int32) if shuffle else np.arange(num_blocks, dtype=np.int32)
    tables = np.full((len(seq_lens), max_blocks), pad, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        tables[b, :n] = perm[off:off + n]
        off += n
    return tables


def slots_for(tables: np.ndarray, b: int, positions: np.ndarray) -> np.ndarray:
    positions = np.asarray(positions, dtype=np.int64)
    return (tables[b, positions // BLOCK_SIZE].astype(np.int64) * BLOCK_SIZE + positions % BLOCK_SIZE).astype(np.int32)


def make_batch(seed: int, seq_lens: Sequence[int], q_lens: Sequence[int], num_q_heads: int,
               num_kv_heads: int, head_dim: int, dtype: str = "bf16",
               num_blocks: Optional[int] = None, max_blocks: Optional[int] = None,
               shuffle: bool = True, scale: Optional[float] = None, name: str = "batch",
               rng: Optional[np.random.Generator] = None, description: str = "",
               values: bool = True, cache: str = "") -> Workload:
    """A single-step varlen batch (``cache="i8"``: bf16 activations over an int8 cache).

    Request b advances ``q_lens[b]`` tokens and then sees ``seq_lens[b]`` keys; its
    first ``seq_lens[b] - q_lens[b]`` tokens are already in the cache.  With ``values=False``
    only lengths, tables and slots are produced (Q/K/V and caches are left empty); they are
    the same as with values, since lengths and placements are drawn first.
    """
    assert dtype in DTYPES
    i8 = cache == "i8"
    assert cache in ("", dtype, "i8") and (not i8 or dtype == "bf16")
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    assert seq_lens.shape == q_lens.shape and seq_lens.ndim == 1
    assert np.all(q_lens >= 1) and np.all(q_lens <= seq_lens)
    rng = rng if rng is not None else np.random.default_rng(seed)
    B = len(seq_lens)
    need = (seq_lens + BLOCK_SIZE - 1) // BLOCK_SIZE
    NB = int(num_blocks) if num_blocks is not None else int(need.sum())
    MB = int(max_blocks) if max_blocks is not None else int(need.max())
    tables = _alloc_blocks(rng, seq_lens, NB, MB, shuffle)

    T = int(q_lens.sum())
    L = int(seq_lens.sum())
    Hq, Hkv, d = num_q_heads, num_kv_heads, head_dim
    if not values:
        slot_mapping = np.empty(T, dtype=np.int32)
        qsl = np.zeros(B + 1, dtype=np.int32)
        t = 0
        for b in range(B):
            s, ql = int(seq_lens[b]), int(q_lens[b])
            slot_mapping[t:t + ql] = slots_for(tables, b, np.arange(s - ql, s))
            t += ql
            qsl[b + 1] = t
        empty = np.zeros((0,), dtype=np_storage_dtype(dtype))
        step = Step(q=empty, k_new=empty, v_new=empty, slot_mapping=slot_mapping,
                    seq_lens=seq_lens.astype(np.int32), query_start_loc=qsl, block_tables=tables)
        return Workload(name=name, dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, num_blocks=NB,
                        scale=float(scale) if scale is not None else 1.0 / math.sqrt(d),
                        k_cache0=empty, v_cache0=empty, steps=[step], seed=seed, description=description,
                        kv_dtype="i8" if i8 else "")
    q = normal_storage(rng, (T, Hq, d), dtype)
    K = normal_storage(rng, (L, Hkv, d), dtype)
    V = normal_storage(rng, (L, Hkv, d), dtype)

    n_ctx = int(np.sum(seq_lens - q_lens))
    if i8:
        kc = np.full((NB, BLOCK_SIZE, Hkv, d), I8_POISON, dtype=np.int8)
        vc = np.full((NB, BLOCK_SIZE, Hkv, d), I8_POISON, dtype=np.int8)
        Kctx = int8_codes(rng, (n_ctx, Hkv, d))
        Vctx = int8_codes(rng, (n_ctx, Hkv, d))
        k_scale = channel_scales(rng, Hkv, d)
        v_scale = channel_scales(rng, Hkv, d)
    else:
        kc, vc = poison_cache((NB, BLOCK_SIZE, Hkv, d), dtype)
    kc2 = kc.reshape(NB * BLOCK_SIZE, Hkv, d)
    vc2 = vc.reshape(NB * BLOCK_SIZE, Hkv, d)
    cpos = 0
    new_rows = np.empty(T, dtype=np.int64)
    slot_mapping = np.empty(T, dtype=np.int32)
    qsl = np.zeros(B + 1, dtype=np.int32)
    lo = 0
    t = 0
    for b in range(B):
        s, ql = int(seq_lens[b]), int(q_lens[b])
        ctx = s - ql
        if ctx > 0:
            sl = slots_for(tables, b, np.arange(ctx))
            if i8:
                kc2[sl] = Kctx[cpos:cpos + ctx]
                vc2[sl] = Vctx[cpos:cpos + ctx]
                cpos += ctx
            else:
                kc2[sl] = K[lo:lo + ctx]
                vc2[sl] = V[lo:lo + ctx]
        slot_mapping[t:t + ql] = slots_for(tables, b, np.arange(ctx, s))
        new_rows[t:t + ql] = np.arange(lo + ctx, lo + s)
        lo += s
        t += ql
        qsl[b + 1] = t
    step = Step(q=q, k_new=np.ascontiguousarray(K[new_rows]), v_new=np.ascontiguousarray(V[new_rows]),
                slot_mapping=slot_mapping, seq_lens=seq_lens.astype(np.int32), query_start_loc=qsl,
                block_tables=tables)
    w = Workload(name=name, dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, num_blocks=NB,
                 scale=float(scale) if scale is not None else 1.0 / math.sqrt(d),
                 k_cache0=kc, v_cache0=vc, steps=[step], seed=seed, description=description)
    if i8:
        w.kv_dtype, w.k_scale, w.v_scale = "i8", k_scale, v_scale
    return w


# ---------------------------------------------------------------------------------------------
# The five synthetic workloads.  Shapes follow the chunked-prefill scenario of P4 (30 decoding
# users + a 30k-token prompt cut into 2048-token chunks), the 16-token blocks of P1 §2.2-2.3, and
# the 32-layer / 32- or 8-KV-head / head_dim-128 model shapes used in P3 §2.3 and §6.3.
# ---------------------------------------------------------------------------------------------

def _sfx(cache: str) -> str:
    return "-i8" if cache == "i8" else ""


def _dsc(cache: str) -> str:
    return ", int8 KV cache with per-(head, channel) scales" if cache == "i8" else ""


def config1(values: bool = True, seed: int = 1) -> Workload:
    """Tiny fp32: 1 sequence, 4 q-heads = 4 KV heads, d=64.  Step 0 prefills 128 tokens,
    steps 1..16 each decode one token (q_len 1, seq_len 128+t).  Scale 1/8; the 9 physical
    blocks are a seeded permutation."""
    rng = np.random.default_rng(seed)
    NB, H, d, S0, ND = 9, 4, 64, 128, 16
    perm = rng.permutation(NB).astype(np.int32)
    tables = perm.reshape(1, NB).copy()
    Q = rng.standard_normal((S0 + ND, H, d), dtype=np.float32)
    K = rng.standard_normal((S0 + ND, H, d), dtype=np.float32)
    V = rng.standard_normal((S0 + ND, H, d), dtype=np.float32)
    kc, vc = poison_cache((NB, BLOCK_SIZE, H, d), "f32")
    steps = []
    rows = np.arange(0, S0)
    steps.append(Step(q=Q[rows].copy(), k_new=K[rows].copy(), v_new=V[rows].copy(),
                      slot_mapping=slots_for(tables, 0, rows), seq_lens=np.array([S0], np.int32),
                      query_start_loc=np.array([0, S0], np.int32), block_tables=tables))
    for t in range(1, ND + 1):
        p = S0 - 1 + t
        rows = np.array([p])
        steps.append(Step(q=Q[rows].copy(), k_new=K[rows].copy(), v_new=V[rows].copy(),
                          slot_mapping=slots_for(tables, 0, rows), seq_lens=np.array([p + 1], np.int32),
                          query_start_loc=np.array([0, 1], np.int32), block_tables=tables))
    return Workload(name="c1_tiny_f32", dtype="f32", num_q_heads=H, num_kv_heads=H, head_dim=d,
                    num_blocks=NB, scale=1.0 / 8.0, k_cache0=kc, v_cache0=vc, steps=steps, seed=seed,
                    description="fp32, 1 seq, 4/4 heads, d=64: prefill 128 then 16 decode steps")


def config2(values: bool = True, seed: int = 2, cache: str = "") -> Workload:
    """Decode batch: 32 requests with q_len 1, contexts U{512..4096}; 32/32 heads, d=128, bf16;
    16384-block pool, shuffled."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(512, 4096, size=32, endpoint=True)
    return make_batch(seed, ctx, np.ones(32, np.int64), 32, 32, 128, "bf16", num_blocks=16384,
                      max_blocks=4096 // BLOCK_SIZE, rng=rng, name="c2_decode_b32" + _sfx(cache), values=values,
                      cache=cache, description="bf16 decode, 32 seqs, 32/32 heads, d=128, ctx U[512,4096], "
                                               "16384-block pool" + _dsc(cache))


def config3(values: bool = True, seed: int = 3, cache: str = "") -> Workload:
    """One-shot causal prefill: S=8192, 32/32 heads, d=128, bf16; 512 blocks, shuffled."""
    rng = np.random.default_rng(seed)
    return make_batch(seed, [8192], [8192], 32, 32, 128, "bf16", num_blocks=512, max_blocks=512,
                      rng=rng, name="c3_prefill_8k" + _sfx(cache), values=values, cache=cache,
                      description="bf16 one-shot causal prefill, S=8192, 32/32 heads, d=128" + _dsc(cache))


def config4(values: bool = True, seed: int = 4, cache: str = "") -> Workload:
    """Mixed chunked-prefill step: 30 decodes (contexts U{1024..8192}) + chunk 15 of a 30720-token
    prompt (2048 new tokens over 28672 cached); 32 q-heads / 8 KV heads, d=128, bf16."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(1024, 8192, size=30, endpoint=True)
    seq = np.concatenate([ctx, [30720]])
    ql = np.concatenate([np.ones(30, np.int64), [2048]])
    nb = int(((ctx + BLOCK_SIZE - 1) // BLOCK_SIZE).sum()) + 30720 // BLOCK_SIZE
    return make_batch(seed, seq, ql, 32, 8, 128, "bf16", num_blocks=nb, max_blocks=30720 // BLOCK_SIZE,
                      rng=rng, name="c4_mixed_chunk" + _sfx(cache), values=values, cache=cache,
                      description="bf16 mixed step: 30 decodes (ctx U[1024,8192]) + 2048-token chunk at 28672 cached, "
                                  "32/8 heads" + _dsc(cache))


def config5(values: bool = True, seed: int = 5, cache: str = "") -> Workload:
    """Length-skewed long decode: 16 requests, contexts log-uniform in [3277, 32768];
    32 q-heads / 8 KV heads, d=128, bf16; pool shuffled so blocks interleave across requests."""
    rng = np.random.default_rng(seed)
    ctx = np.clip(np.round(np.exp(rng.uniform(math.log(3277), math.log(32768), size=16))), 3277, 32768).astype(np.int64)
    nb = int(((ctx + BLOCK_SIZE - 1) // BLOCK_SIZE).sum())
    return make_batch(seed, ctx, np.ones(16, np.int64), 32, 8, 128, "bf16", num_blocks=nb,
                      max_blocks=32768 // BLOCK_SIZE, rng=rng, name="c5_skewed_decode" + _sfx(cache), values=values,
                      cache=cache, description="bf16 decode, 16 seqs, ctx log-U[3277,32768], 32/8 heads, "
                                               "interleaved blocks" + _dsc(cache))


CONFIGS = {"c1": config1, "c2": config2, "c3": config3, "c4": config4, "c5": config5}


def verify_variant(w: Workload, k: int) -> Workload:
    """A decode workload turned into a verification step: each request's last k tokens are the
    step's new tokens (q_len = k, same seq_len), the rest stays cached.  Same seed and draw order
    as the decode workload (lengths and placements identical)."""
    st = w.steps[0]
    assert len(w.steps) == 1 and np.all(st.q_lens == 1)
    B = st.num_seqs
    q_lens = np.minimum(k, st.seq_lens.astype(np.int64))
    v = make_batch(w.seed, st.seq_lens, q_lens, w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype,
                   num_blocks=w.num_blocks, max_blocks=st.block_tables.shape[1], rng=_replay_rng(w),
                   name=f"{w.name}-v{k}", description=w.description + f", verifying {k} tokens per request",
                   cache=w.kv_dtype)
    assert v.steps[0].num_seqs == B
    return v


def _replay_rng(w: Workload) -> np.random.Generator:
    """The generator state a config function hands to make_batch (it draws the lengths first)."""
    rng = np.random.default_rng(w.seed)
    name = w.name.split("-")[0]
    if name == "c2_decode_b32":
        rng.integers(512, 4096, size=32, endpoint=True)
    elif name == "c5_skewed_decode":
        rng.uniform(math.log(3277), math.log(32768), size=16)
    else:
        raise ValueError(f"no verify variant for {w.name}")
    return rng


def chunked_steps(w: Workload, chunk_sizes: Sequence[int]) -> Workload:
    """Re-express a single-request prefill workload (q_len == seq_len) as successive chunks.

    Chunk i appends tokens [c_i, c_i + n_i) and attends with q_len = n_i over seq_len = c_i + n_i
    (P4 "把长输入切成块": each chunk reads the KV already cached, then writes its own)."""
    assert len(w.steps) == 1
    st = w.steps[0]
    assert st.num_seqs == 1 and int(st.q_lens[0]) == int(st.seq_lens[0])
    S = int(st.seq_lens[0])
    assert sum(chunk_sizes) == S
    steps = []
    c = 0
    for n in chunk_sizes:
        rows = np.arange(c, c + n)
        steps.append(Step(q=st.q[rows].copy(), k_new=st.k_new[rows].copy(), v_new=st.v_new[rows].copy(),
                          slot_mapping=st.slot_mapping[rows].copy(), seq_lens=np.array([c + n], np.int32),
                          query_start_loc=np.array([0, n], np.int32), block_tables=st.block_tables))
        c += n
    return Workload(name=w.name + "_chunked", dtype=w.dtype, num_q_heads=w.num_q_heads,
                    num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, num_blocks=w.num_blocks, scale=w.scale,
                    k_cache0=w.k_cache0, v_cache0=w.v_cache0, steps=steps, seed=w.seed,
                    description=w.description + f" as chunks {list(chunk_sizes)}",
                    kv_dtype=w.kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale)
