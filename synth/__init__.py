"""Seeded synthetic inputs for split-KV decode attention.

This module only draws and encodes input tensors (queries, a key/value cache,
sequence lengths, block tables).  It holds none of the attention arithmetic,
so that both the GPU library's tests and the fp64 oracle can consume the same
inputs without sharing any code of the method itself.

Generator: numpy PCG64, one independent stream per tensor, standard normal
fp32 draws rounded to the storage type (IEEE binary16 via numpy, bfloat16 by
explicit round-to-nearest-even on the fp32 bit pattern).  The rounded values
are what both sides read, so no side sees a value the other does not.

Seeds: q=1, K=2, V=3 (the handbook's paged decode example fills q, K and V
from seeds 1, 2 and 3), block-table permutation=7 (that example shuffles the
physical blocks with seed 7), sequence lengths=11, stress mask=13.

Storage conventions (what the arrays hold):
  f32  -> numpy float32
  f16  -> numpy float16
  bf16 -> numpy uint16 holding the bfloat16 bit pattern
  fp8  -> numpy uint8 holding an OCP FP8 E4M3 bit pattern (K and V only; q
          is bf16).  A cache tensor with scale c stores x / c rounded to
          nearest even and saturated at +-448, for the N(0, 1) draw x; the
          value it stands for is stored * c.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

SEED_Q, SEED_K, SEED_V, SEED_PERM, SEED_LENS, SEED_STRESS = 1, 2, 3, 7, 11, 13

DTYPES = ("f32", "f16", "bf16", "fp8")
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3}
E4M3_MAX = 448.0
E4M3_QNAN = 0x7F
BF16_QNAN = 0x7FC0
F16_QNAN = 0x7E00


# --------------------------------------------------------------------------
# encodings
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 -> bfloat16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_QNAN
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP FP8 E4M3 bits, nearest even, saturated at +-448 (torch's encoder)."""
    import torch
    x = np.clip(np.ascontiguousarray(x, dtype=np.float32), -E4M3_MAX, E4M3_MAX)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of E4M3 bits to fp32 (torch's decoder)."""
    import torch
    b = np.ascontiguousarray(b, dtype=np.uint8)
    return torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float32).numpy()


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 values -> storage array of `dtype` (rounded to nearest even)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "fp8":
        return f32_to_e4m3_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def decode_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> exact float64 values (for building expected shapes in tests).
    For fp8 this is the stored value, before the tensor's scale."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    if dtype == "fp8":
        return e4m3_bits_to_f32(a).astype(np.float64)
    return np.asarray(a).astype(np.float64)


def nan_value(dtype: str):
    return {"f32": np.float32(np.nan), "f16": np.float16(np.nan), "bf16": np.uint16(BF16_QNAN),
            "fp8": np.uint8(E4M3_QNAN)}[dtype]


_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8": np.uint8}
_CHUNK = 1 << 20


def normal(seed: int, shape, dtype: str, scale=1.0) -> np.ndarray:
    """Standard normal draws from PCG64(seed), rounded to `dtype` storage
    (fp8: the draw divided by `scale`, see the module docstring; `scale` may
    also be one value per KV head, shape[-2] of them, for per-head scales).

    Drawn in chunks through reused buffers (one pass over the output, no
    full-size temporaries); the values are the generator's sequence in order.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.empty(shape, dtype=_STORAGE[dtype])
    flat = out.reshape(-1)
    n = flat.size
    buf = np.empty(min(_CHUNK, max(n, 1)), dtype=np.float32)
    u = buf.view(np.uint32)
    t = np.empty_like(u)
    for i in range(0, n, _CHUNK):
        m = min(_CHUNK, n - i)
        rng.standard_normal(out=buf[:m], dtype=np.float32)
        if dtype == "bf16":
            # round to nearest even on the fp32 bits (normal draws are never NaN)
            tm, um = t[:m], u[:m]
            np.right_shift(um, 16, out=tm)
            np.bitwise_and(tm, 1, out=tm)
            np.add(tm, 0x7FFF, out=tm)
            np.add(tm, um, out=tm)
            np.right_shift(tm, 16, out=tm)
            flat[i:i + m] = tm
        elif dtype == "fp8":
            if np.ndim(scale) == 0:
                flat[i:i + m] = f32_to_e4m3_bits(buf[:m] / np.float32(scale))
            else:   # element j belongs to KV head (j // d) % Hkv
                heads = (np.arange(i, i + m, dtype=np.int64) // shape[-1]) % shape[-2]
                flat[i:i + m] = f32_to_e4m3_bits(buf[:m] / np.asarray(scale, np.float32)[heads])
        else:
            flat[i:i + m] = buf[:m]
    return out


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    """Shape and recipe of one decode-attention problem."""
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    dtype: str
    split: int
    N: int                      # cache capacity per request (contiguous) / max length (paged)
    len_range: Optional[tuple] = None   # (lo, hi) inclusive uniform lengths; None -> every length = N
    page_size: int = 0          # 0 -> contiguous [B, N, Hkv, d]; else paged [P, page, Hkv, d]
    stress_frac: float = 0.0    # Bernoulli fraction of key rows (b, t, kvh) scaled by stress_scale
    stress_scale: float = 8.0
    fixed_lens: Optional[tuple] = None  # explicit per-request lengths (overrides len_range)
    qdtype: Optional[str] = None        # storage of q; None -> dtype (bf16 for an fp8 cache)
    k_scale: float = 1.0                # fp8 caches: a stored K value stands for stored * k_scale
    v_scale: float = 1.0
    q_len: int = 1                      # query tokens per request: q [B, q_len, Hq, d]
    k_scales: Optional[tuple] = None    # fp8 caches: one K scale per KV head, replacing k_scale
    v_scales: Optional[tuple] = None    # fp8 caches: one V scale per KV head, replacing v_scale

    @property
    def q_dtype(self) -> str:
        if self.qdtype is not None:
            return self.qdtype
        return "bf16" if self.dtype == "fp8" else self.dtype

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_splits(self) -> int:
        return -(-self.N // self.split)

    @property
    def max_blocks(self) -> int:
        return -(-self.N // self.page_size) if self.page_size else 0


WORKLOADS = {
    "tiny_mha": Workload("tiny_mha", B=1, Hq=8, Hkv=8, d=64, dtype="f32", split=128, N=512),
    "llama2_7b_mha": Workload("llama2_7b_mha", B=1, Hq=32, Hkv=32, d=128, dtype="f16", split=256, N=4096),
    "long_gqa_32k": Workload("long_gqa_32k", B=1, Hq=32, Hkv=8, d=128, dtype="bf16", split=256, N=32768),
    "paged_batched_gqa": Workload("paged_batched_gqa", B=64, Hq=64, Hkv=8, d=128, dtype="bf16", split=256,
                                  N=16384, len_range=(1024, 16384), page_size=16),
    # a batch of short requests that fills the GPU many times over (256 x 8 KV heads): the split
    # heuristic's one split per row (1008 tokens, page-aligned), where AUTO writes the result from
    # the partial kernel with no merge (the Flash-Decoding page's no-split rule)
    "paged_batch_short": Workload("paged_batch_short", B=256, Hq=32, Hkv=8, d=128, dtype="bf16", split=1008,
                                  N=1008, len_range=(1, 1000), page_size=16),
    # no split size is given for this shape: 1024 is what the library's split heuristic picks for it
    "umax_stress": Workload("umax_stress", B=4, Hq=64, Hkv=8, d=128, dtype="bf16", split=1024, N=131072,
                            stress_frac=0.02, stress_scale=8.0),
    # a whole 4k prompt as queries (prefill): every token attends causally to
    # the tokens up to it; one split per query tile (the tiles alone fill the GPU)
    "prefill_gqa_4k": Workload("prefill_gqa_4k", B=1, Hq=32, Hkv=8, d=128, dtype="bf16", split=4096, N=4096,
                               q_len=4096),
    # the long-context GQA shape with an 8-bit cache (scale 1/64: N(0, 1) draws stored as 64 x)
    "long_gqa_32k_fp8": Workload("long_gqa_32k_fp8", B=1, Hq=32, Hkv=8, d=128, dtype="fp8", split=256,
                                 N=32768, k_scale=1.0 / 64, v_scale=1.0 / 64),
    # the same with one scale per KV head (distinct, not powers of two)
    "long_gqa_32k_fp8_head_scales": Workload(
        "long_gqa_32k_fp8_head_scales", B=1, Hq=32, Hkv=8, d=128, dtype="fp8", split=256, N=32768,
        k_scales=tuple(c / 64 for c in (0.75, 1.25, 0.9, 1.1, 0.8, 1.2, 0.95, 1.05)),
        v_scales=tuple(c / 64 for c in (1.3, 0.7, 1.15, 0.85, 1.05, 0.95, 0.6, 1.4))),
    # the long-context GQA shape verifying 4 drafted tokens (4 x 4 query rows per KV head)
    "long_gqa_32k_verify4": Workload("long_gqa_32k_verify4", B=1, Hq=32, Hkv=8, d=128, dtype="bf16", split=256,
                                     N=32768, q_len=4),
    # the same with 8 drafted tokens: 32 query rows per KV head, two 16-row tiles
    "long_gqa_32k_verify8": Workload("long_gqa_32k_verify8", B=1, Hq=32, Hkv=8, d=128, dtype="bf16", split=256,
                                     N=32768, q_len=8),
}


def seq_lens_for(w: Workload) -> np.ndarray:
    if w.fixed_lens is not None:
        lens = np.asarray(w.fixed_lens, dtype=np.int32)
        assert lens.shape == (w.B,)
        return lens
    if w.len_range is None:
        return np.full(w.B, w.N, dtype=np.int32)
    lo, hi = w.len_range
    rng = np.random.Generator(np.random.PCG64(SEED_LENS))
    return rng.integers(lo, hi, size=w.B, endpoint=True).astype(np.int32)


def block_table_for(w: Workload, lens: np.ndarray):
    """Physical pages assigned request by request from a seeded permutation.

    Returns (block_table int32 [B, max_blocks] with unused entries -1, P).
    """
    pages_per = (lens.astype(np.int64) + w.page_size - 1) // w.page_size
    P = int(pages_per.sum())
    rng = np.random.Generator(np.random.PCG64(SEED_PERM))
    perm = rng.permutation(P).astype(np.int32)
    table = np.full((w.B, w.max_blocks), -1, dtype=np.int32)
    nxt = 0
    for b in range(w.B):
        n = int(pages_per[b])
        table[b, :n] = perm[nxt:nxt + n]
        nxt += n
    return table, P


@dataclass
class Inputs:
    w: Workload
    q: np.ndarray            # [B, Hq, d]
    k: np.ndarray            # contiguous [B, N, Hkv, d] or paged [P, page, Hkv, d]
    v: np.ndarray
    seq_lens: np.ndarray     # int32 [B]
    block_table: Optional[np.ndarray] = None   # int32 [B, max_blocks]
    stress_mask: Optional[np.ndarray] = None   # bool, same leading shape as k[..., 0]

    @property
    def kv_bytes(self) -> int:
        """Bytes of K and V for every (b, kv head, valid token), counted once."""
        w = self.w
        return int(self.seq_lens.astype(np.int64).sum()) * w.Hkv * w.d * ELEM_BYTES[w.dtype] * 2


def make_inputs(w: Workload, poison_tail: bool = True) -> Inputs:
    """Draw the seeded inputs of workload `w`.

    With poison_tail, every cache slot that no valid token occupies (tokens past
    seq_len in a contiguous cache, the unused slots of a request's last page) is
    set to NaN, so that a kernel that reads or weights them shows it.
    """
    lens = seq_lens_for(w)
    q = normal(SEED_Q, (w.B, w.q_len, w.Hq, w.d) if w.q_len > 1 else (w.B, w.Hq, w.d), w.q_dtype)
    table = None
    if w.page_size:
        table, P = block_table_for(w, lens)
        shape = (P, w.page_size, w.Hkv, w.d)
    else:
        shape = (w.B, w.N, w.Hkv, w.d)
    k = normal(SEED_K, shape, w.dtype, w.k_scales if w.k_scales is not None else w.k_scale)
    v = normal(SEED_V, shape, w.dtype, w.v_scales if w.v_scales is not None else w.v_scale)

    mask = None
    if w.stress_frac > 0:
        rng = np.random.Generator(np.random.PCG64(SEED_STRESS))
        mask = rng.random(size=shape[:3]) < w.stress_frac
        rows = decode_f64(k[mask], w.dtype).astype(np.float32)
        k[mask] = encode(rows * np.float32(w.stress_scale), w.dtype)   # exact: power-of-two scale

    if poison_tail:
        nanv = nan_value(w.dtype)
        for b in range(w.B):
            n = int(lens[b])
            if w.page_size:
                if n % w.page_size:
                    last = table[b, n // w.page_size]
                    k[last, n % w.page_size:] = nanv
                    v[last, n % w.page_size:] = nanv
            elif n < w.N:
                k[b, n:] = nanv
                v[b, n:] = nanv
    return Inputs(w, q, k, v, lens, table, mask)


def with_lens(w: Workload, lens, name: Optional[str] = None) -> Workload:
    """Same workload with explicit per-request lengths (B taken from len(lens))."""
    lens = tuple(int(x) for x in lens)
    N = max(max(lens), 1)
    if w.page_size:
        N = -(-N // w.page_size) * w.page_size
    return replace(w, name=name or w.name, B=len(lens), N=N, fixed_lens=lens, len_range=None)


def small(w: Workload, **kw) -> Workload:
    """A reduced copy of a workload (for quick parity cases)."""
    return replace(w, **kw)
