"""Seeded synthetic workloads for MoE routing, dispatch and combine.

This module only draws random inputs; it holds none of the method's
arithmetic, and both the HIP library's callers and the CPU oracle's callers
take their inputs from it.

Shapes follow the test settings the DeepEP pages describe: the normal
(training / prefill) kernels at 4096 tokens per batch, hidden 7168, top-4
groups, top-8 experts, FP8 dispatch and BF16 combine, and the low-latency
(decode) kernels at 128 tokens per batch, hidden 7168, top-8 experts ([NEWS]
"具体性能方面", [DAY2] "DeepEP 的性能表现", [DE]).  Expert counts, group
counts, value distributions, skew and outliers are readings (the pages do not
give them): 256 experts in 8 groups as in DeepSeek-V3, logits ~ N(0, 1),
hidden states ~ N(0, 1), and 32 virtual expert ranks of 8 experts.

Random streams: numpy PCG64 seeded through SeedSequence(seed).spawn(4), one
child each for x, logits, expert outputs y and the per-expert bias.
bf16 arrays are the upper 16 bits of fp32 draws (truncation), returned as
uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens
    H: int            # hidden size (multiple of 128)
    E: int            # experts
    G: int            # expert groups
    TG: int           # groups kept per token
    k: int            # experts per token
    R: int            # virtual expert ranks
    m: int = 0        # scores summed per group score (0 -> k // TG)
    seed: int = 0
    skew: str = "none"        # "none" | "zipf_rank" | "zipf_iid"
    outlier_frac: float = 0.0  # fraction of hidden channels scaled x100

    @property
    def topm(self) -> int:
        return self.m or max(1, self.k // self.TG)

    @property
    def nrows(self) -> int:
        return self.T * self.k

    # algorithmic bytes (each byte the step must move once)
    def bytes_dispatch_fp8(self) -> int:
        return self.T * (2 * self.H + self.k * self.H + 4 * self.k * (self.H // 128) + 4 * self.k)

    def bytes_dispatch_bf16(self) -> int:
        return self.T * (2 * self.H + 2 * self.k * self.H + 4 * self.k)

    def bytes_combine(self) -> int:
        return self.T * (2 * self.k * self.H + 2 * self.H + 8 * self.k)

    def bytes_route(self) -> int:
        return self.T * (4 * self.E + 8 * self.k)

    def bytes_layout(self) -> int:
        # read topk_idx, write slot and recv_token (counts/offsets are O(E))
        return self.T * self.k * 12 + 4 * (2 * self.E + 1 + self.R)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


TINY = Workload("tiny", T=64, H=256, E=16, G=4, TG=2, k=4, R=4, seed=20260)
DECODE = Workload("decode", T=128, H=7168, E=256, G=8, TG=8, k=8, R=32, seed=20261)
PREFILL = Workload("prefill", T=4096, H=7168, E=256, G=8, TG=4, k=8, R=32, seed=20262)
SKEWED = Workload("skewed", T=4096, H=7168, E=256, G=8, TG=4, k=8, R=32, seed=20263,
                  skew="zipf_rank")
LARGE = Workload("large", T=16384, H=7168, E=256, G=8, TG=4, k=8, R=32, seed=20264,
                 outlier_frac=0.01)
# literal reading of "Zipf(1.2) * 3" per-expert bias: heavy ties, every token
# routed alike; kept as a stress case for contention and tie-breaking
SKEWED_LITERAL = SKEWED.replace(name="skewed_literal", skew="zipf_iid", seed=20265)

CONFIGS = {w.name: w for w in (TINY, DECODE, PREFILL, SKEWED, LARGE, SKEWED_LITERAL)}


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(4)]


def _to_bf16_bits(f32: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(f32, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def gen_x(w: Workload, T: int | None = None) -> np.ndarray:
    """Hidden states, bf16 bits [T, H] ~ N(0,1); with outlier_frac > 0,
    round(frac * H) channels (seeded choice) are multiplied by 100 in fp32
    before conversion."""
    T = w.T if T is None else T
    rx = _streams(w.seed)[0]
    x = rx.standard_normal((T, w.H), dtype=np.float32)
    if w.outlier_frac > 0:
        n_out = int(round(w.outlier_frac * w.H))
        ch = _streams(w.seed)[3].choice(w.H, size=n_out, replace=False)
        x[:, ch] *= np.float32(100.0)
    return _to_bf16_bits(x)


def expert_bias(w: Workload) -> np.ndarray | None:
    rb = _streams(w.seed)[3]
    if w.skew == "none":
        return None
    if w.skew == "zipf_rank":
        # Zipf rank profile: expert with rank r (a seeded permutation of 1..E)
        # gets 3 * r^-1.2
        ranks = rb.permutation(w.E) + 1
        return (3.0 * ranks.astype(np.float64) ** -1.2).astype(np.float32)
    if w.skew == "zipf_iid":
        return (rb.zipf(1.2, size=w.E).astype(np.float64) * 3.0).astype(np.float32)
    raise ValueError(w.skew)


def gen_logits(w: Workload, T: int | None = None) -> np.ndarray:
    """Router logits fp32 [T, E] ~ N(0,1), plus the per-expert bias of the
    skewed workloads (added in fp32)."""
    T = w.T if T is None else T
    rl = _streams(w.seed)[1]
    lg = rl.standard_normal((T, w.E), dtype=np.float32)
    b = expert_bias(w)
    if b is not None:
        lg = (lg + b[None, :]).astype(np.float32)
    return lg


def gen_y(w: Workload, nrows: int | None = None, chunk_rows: int = 8192) -> np.ndarray:
    """Synthetic expert outputs, bf16 bits [nrows, H] ~ N(0,1), one row per
    receive row (the expert computation itself is out of scope)."""
    nrows = w.nrows if nrows is None else nrows
    ry = _streams(w.seed)[2]
    out = np.empty((nrows, w.H), np.uint16)
    for r0 in range(0, nrows, chunk_rows):
        r1 = min(nrows, r0 + chunk_rows)
        out[r0:r1] = _to_bf16_bits(ry.standard_normal((r1 - r0, w.H), dtype=np.float32))
    return out


def sha256(a: np.ndarray) -> str:
    """SHA-256 of an array's bytes in C order (hex digest)."""
    return hashlib.sha256(memoryview(np.ascontiguousarray(a)).cast("B")).hexdigest()
