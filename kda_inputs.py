"""Seeded synthetic inputs for the KDA decode workloads.

This module only draws numbers; it holds none of the update's arithmetic.
Both the CPU oracle (through the tests) and the HIP library (through the
tests and the benchmark) receive the very same host arrays from here.

Recipe (NumPy PCG64, ``np.random.default_rng(seed)``), drawn in this order:
  1. initial pool S0 [n_slots, H, K, V] ~ N(0, 0.05^2) in fp32;
  2. q, k, v [R, H, K] ~ N(0, 1) (fp32);
  3. g_raw [R, H, K] ~ N(0, 1); g = -softplus(g_raw) = -log(1 + e^g_raw),
     the per-key-channel log-decay, so a = e^g lies in (0, 1);
  4. b [R, H] ~ N(0, 1), the gate logit (beta = sigmoid(b));
  5. slot ids: the first R entries of a permutation of the pool's slots.
An fp16 pool is the fp32 draw rounded to nearest even (NumPy's float16 cast)
and kept as its uint16 bit patterns.  R = n_req * n_rows; the rows of one
request are adjacent.

The named workloads mirror the shapes the pages discuss for Kimi-K3's KDA
layers (H = 12 heads of K = V = 128 per rank; N = 64 decode slots; 1 + 7
speculative rows; 69 KDA layers): see ROCm/ATOM PR #2130 (What, Memory) and
ROCm/ATOM PR #2945 (Method: 7 speculative tokens).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

H_DEFAULT = 12
K_DEFAULT = 128
V_DEFAULT = 128
S0_STD = 0.05


@dataclass
class DecodeInputs:
    """One decode launch's worth of host inputs."""
    name: str
    dtype: str                 # "f32" or "f16": the pool's element type
    pool: np.ndarray           # [n_slots, H, K, V] float32, or uint16 fp16 bits
    slot_ids: np.ndarray       # int32 [R]
    q: np.ndarray              # float32 [R, H, K]
    k: np.ndarray
    v: np.ndarray              # float32 [R, H, V]
    g: np.ndarray              # float32 [R, H, K] (log-decay, <= 0)
    b: np.ndarray              # float32 [R, H]
    n_rows: int
    scale: float
    meta: dict = field(default_factory=dict)

    @property
    def n_req(self) -> int:
        return self.slot_ids.size // self.n_rows

    @property
    def shape(self):
        return self.pool.shape

    def state_bytes(self) -> int:
        """Algorithmic state bytes of the launch: each request's tile is read
        once and written once per row."""
        _, H, K, V = self.pool.shape
        elem = 4 if self.dtype == "f32" else 2
        return self.n_req * H * K * V * elem * (1 + self.n_rows)

    def io_bytes(self) -> int:
        """Bytes of the per-row vectors: q, k, g, v and out (fp32), b, ids."""
        R = self.slot_ids.size
        _, H, K, V = self.pool.shape
        return R * H * (3 * K + 2 * V + 1) * 4 + R * 4


def draw_pool(rng: np.random.Generator, n_slots: int, H: int, K: int, V: int,
              dtype: str, std: float = S0_STD) -> np.ndarray:
    s0 = rng.standard_normal((n_slots, H, K, V), dtype=np.float32)
    s0 *= np.float32(std)
    if dtype == "f32":
        return s0
    if dtype == "f16":
        return s0.astype(np.float16).view(np.uint16)
    raise ValueError("pool dtype must be 'f32' or 'f16'")


def draw_rows(rng: np.random.Generator, R: int, H: int, K: int, V: int):
    q = rng.standard_normal((R, H, K), dtype=np.float32)
    k = rng.standard_normal((R, H, K), dtype=np.float32)
    v = rng.standard_normal((R, H, V), dtype=np.float32)
    g_raw = rng.standard_normal((R, H, K), dtype=np.float32).astype(np.float64)
    g = (-np.logaddexp(0.0, g_raw)).astype(np.float32)
    b = rng.standard_normal((R, H), dtype=np.float32)
    return q, k, v, g, b


def make_inputs(name: str, n_slots: int, n_req: int, n_rows: int,
                dtype: str = "f32", H: int = H_DEFAULT, K: int = K_DEFAULT,
                V: int = V_DEFAULT, seed: int = 0) -> DecodeInputs:
    if n_req * n_rows > n_slots:
        raise ValueError("need n_req * n_rows distinct slots")
    rng = np.random.default_rng(seed)
    pool = draw_pool(rng, n_slots, H, K, V, dtype)
    R = n_req * n_rows
    q, k, v, g, b = draw_rows(rng, R, H, K, V)
    slot_ids = rng.permutation(n_slots)[:R].astype(np.int32)
    return DecodeInputs(name=name, dtype=dtype, pool=pool, slot_ids=slot_ids,
                        q=q, k=k, v=v, g=g, b=b, n_rows=n_rows,
                        scale=float(1.0 / np.sqrt(K)))


# The named workloads ------------------------------------------------------

def single_slot_f32(seed: int = 0) -> DecodeInputs:
    """One slot, one token, fp32 pool, H=12, K=V=128."""
    return make_inputs("single-slot decode, fp32 pool, H=12 K=V=128", 1, 1, 1, "f32", seed=seed)


def batched_f32(seed: int = 0) -> DecodeInputs:
    """64 slots gathered from a 96-slot pool, one token each, fp32 pool."""
    return make_inputs("batched decode N=64 of 96 slots, fp32 pool, H=12 K=V=128", 96, 64, 1, "f32", seed=seed)


def batched_f16(seed: int = 0) -> DecodeInputs:
    """As batched_f32 with an fp16 pool."""
    return make_inputs("batched decode N=64 of 96 slots, fp16 pool, H=12 K=V=128", 96, 64, 1, "f16", seed=seed)


def spec_verify_f16(seed: int = 0) -> DecodeInputs:
    """8 requests x (1 + 7 draft) rows, fp16 pool of 96 slots; 64 snapshot
    slots, each request's initial state in its row-0 slot."""
    return make_inputs("spec-verify 8 req x 8 rows, fp16 pool of 96 slots, H=12 K=V=128", 96, 8, 8, "f16", seed=seed)


def drift_tokens(n_tokens: int, seed: int = 0, H: int = H_DEFAULT, K: int = K_DEFAULT,
                 V: int = V_DEFAULT):
    """Long single-slot run: the initial fp32 state S0 [1, H, K, V] and fresh
    per-token inputs q, k, v, g [T, H, *], b [T, H] (one row per launch)."""
    rng = np.random.default_rng(seed)
    s0 = draw_pool(rng, 1, H, K, V, "f32")
    q, k, v, g, b = draw_rows(rng, n_tokens, H, K, V)
    return s0, q, k, v, g, b


def layer_step(layer: int, dtype: str, n_slots: int = 64, H: int = H_DEFAULT) -> DecodeInputs:
    """One of the 69 KDA layers of a full decode step: its own 64-slot pool,
    64 requests x 1 token; seed = layer index."""
    return make_inputs("layer %d of a 69-layer step, %s pool" % (layer, dtype),
                       n_slots, n_slots, 1, dtype, H=H, seed=layer)


WORKLOADS = {
    "single_f32": single_slot_f32,
    "batched_f32": batched_f32,
    "batched_f16": batched_f16,
    "spec_verify_f16": spec_verify_f16,
}


@dataclass
class ConvInputs:
    """Inputs of a decode launch with the short convolution fused in front:
    the decode inputs (q, k, v unused) plus the conv history pool (bfloat16
    bits [n_slots, 3, 3, H, 128]), the raw q|k|v rows x [R, 3, H, 128] and the
    taps w [3, H, 128, 4]."""
    dec: DecodeInputs
    conv: np.ndarray
    x: np.ndarray
    w: np.ndarray


def make_conv_inputs(name: str, n_slots: int, n_req: int, n_rows: int, dtype: str = "f32",
                     H: int = H_DEFAULT, seed: int = 0) -> ConvInputs:
    """Recipe: the decode draws of make_inputs(seed), then from
    default_rng(seed + 10**6): the conv history ~ N(0, 1) cut to bfloat16 (the
    top 16 bits of the fp32 draw: any bfloat16 value is a valid history), the
    raw rows x ~ N(0, 1), the taps w ~ N(0, 0.5^2)."""
    dec = make_inputs(name, n_slots, n_req, n_rows, dtype, H=H, seed=seed)
    rng = np.random.default_rng(seed + 10 ** 6)
    hist = rng.standard_normal((n_slots, 3, 3, H, K_DEFAULT), dtype=np.float32)
    conv = (hist.view(np.uint32) >> 16).astype(np.uint16)
    R = n_req * n_rows
    x = rng.standard_normal((R, 3, H, K_DEFAULT), dtype=np.float32)
    w = rng.standard_normal((3, H, K_DEFAULT, 4), dtype=np.float32) * np.float32(0.5)
    return ConvInputs(dec, conv, x, w)


@dataclass
class PrefillInputs:
    """Inputs of one prefill launch: n_seq sequences packed along the token
    axis (cu_seqlens), each starting from its initial slot of the pool and
    storing its final state to its destination slot."""
    name: str
    dtype: str
    pool: np.ndarray           # [n_slots, H, K, V] float32, or uint16 fp16 bits
    init_slot_ids: np.ndarray  # int32 [n_seq]
    dst_slot_ids: np.ndarray   # int32 [n_seq]
    cu_seqlens: np.ndarray     # int32 [n_seq + 1]
    q: np.ndarray              # float32 [T, H, K]
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    b: np.ndarray              # float32 [T, H]
    scale: float

    @property
    def n_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    def io_bytes(self) -> int:
        """Algorithmic bytes: q, k, v, g, out (fp32) and b per token-head,
        each sequence's state read once and written once, the id tables."""
        _, H, K, V = self.pool.shape
        elem = 4 if self.dtype == "f32" else 2
        n_seq = self.init_slot_ids.size
        return (self.n_tokens * H * (3 * K + 2 * V + 1) * 4 + 2 * n_seq * H * K * V * elem
                + 4 * (3 * n_seq + 1))


def make_prefill_inputs(name: str, lengths, n_slots: int, dtype: str = "f32", H: int = H_DEFAULT,
                        K: int = K_DEFAULT, V: int = V_DEFAULT, seed: int = 0,
                        in_place: bool = True) -> PrefillInputs:
    """Recipe: default_rng(seed) draws the pool S0 ~ N(0, 0.05^2), then the
    rows q, k, v, g, b of all T = sum(lengths) tokens as for decode, then a
    permutation of the pool's slots: the first n_seq are the initial slots,
    the next n_seq the destination slots (unless in_place)."""
    lengths = [int(x) for x in lengths]
    n_seq = len(lengths)
    if n_seq * (1 if in_place else 2) > n_slots:
        raise ValueError("not enough slots")
    rng = np.random.default_rng(seed)
    pool = draw_pool(rng, n_slots, H, K, V, dtype)
    T = sum(lengths)
    q, k, v, g, b = draw_rows(rng, T, H, K, V)
    perm = rng.permutation(n_slots).astype(np.int32)
    init = perm[:n_seq].copy()
    dst = init.copy() if in_place else perm[n_seq:2 * n_seq].copy()
    cu = np.zeros(n_seq + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    return PrefillInputs(name=name, dtype=dtype, pool=pool, init_slot_ids=init, dst_slot_ids=dst,
                         cu_seqlens=cu, q=q, k=k, v=v, g=g, b=b, scale=float(1.0 / np.sqrt(K)))


def prefill_lengths(n_seq: int, mean: int, seed: int) -> list:
    """A ragged length mix: uniform on [mean/4, 7*mean/4], so the total is
    about n_seq * mean and the lengths mostly fall between chunk boundaries."""
    rng = np.random.default_rng(seed + 7)
    return [int(x) for x in rng.integers(max(1, mean // 4), 7 * mean // 4 + 1, size=n_seq)]


def prefill_batch(dtype: str, seed: int = 0) -> PrefillInputs:
    """The prefill workload: 32 prompts of ragged length (mean 1024 tokens,
    about 32K tokens in all), H = 12, K = V = 128, each from its own slot of
    a 64-slot pool, final state stored in place."""
    return make_prefill_inputs("prefill 32 prompts x ~1K tokens (ragged), %s pool, H=12 K=V=128"
                               % dtype, prefill_lengths(32, 1024, seed), 64, dtype, seed=seed)
