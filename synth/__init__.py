"""Seeded synthetic inputs for the paged decode-attention path.

Shared by the tests, the smoke check and the benchmark, on both sides of every
comparison (the CPU oracle and the HIP library). It holds none of the method's
arithmetic: only random draws, the construction of context lengths, block tables,
page lists and slot mappings, and the shapes of the benchmarked workloads.

Recipe:
  * Q, K, V ~ N(0, 1), drawn in fp32 from a torch generator seeded by a tuple
    (workload seed, layer, sequence, tensor tag), then rounded to nearest even
    into the cache dtype. A logical token's K/V values depend only on that tuple
    and its position, never on where its page is placed.
  * Context lengths ~ uniform integers in [lo, hi].
  * Block tables: the pool holds sum_b ceil(L_b / P) blocks (plus any spare
    blocks); a seeded random permutation of the block ids is dealt out to the
    sequences in order, so placement is random and every sequence owns its pages.
  * Page lists: per sequence, the page holding the newest token plus k-1 distinct
    earlier pages drawn without replacement, sorted ascending.
"""
from __future__ import annotations

import dataclasses
from typing import Sequence

import torch

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}

_MASK64 = (1 << 64) - 1


def _mix(z: int) -> int:
    # splitmix64 finaliser: decorrelates nearby seed tuples
    z = (z + 0x9E3779B97F4A7C15) & _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def seed_of(*parts) -> int:
    h = 0x5EED0000
    for p in parts:
        if isinstance(p, str):
            raw = p.encode()
            words = [int.from_bytes(raw[i:i + 8].ljust(8, b"\0"), "little")
                     for i in range(0, max(len(raw), 1), 8)]
            for wd in words + [len(raw)]:
                h = _mix(h ^ wd)
            continue
        h = _mix(h ^ (int(p) & _MASK64))
    return h & ((1 << 63) - 1)


def generator(*parts, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*parts))
    return g


def normal(shape: Sequence[int], *parts, dtype: str = "bf16", device="cpu",
           std: float = 1.0) -> torch.Tensor:
    """N(0, std^2) drawn in fp32, rounded to nearest even into `dtype`."""
    g = generator(*parts, device=device)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(TORCH_DTYPE[dtype])


def uniform_lengths(batch: int, lo: int, hi: int, *parts) -> torch.Tensor:
    g = generator("lens", *parts)
    return torch.randint(lo, hi + 1, (batch,), generator=g, dtype=torch.int64).to(torch.int32)


def blocks_needed(lens, P: int) -> list[int]:
    return [(int(L) + P - 1) // P for L in lens]


def block_tables(lens, P: int, *parts, spare_blocks: int = 0, max_blocks: int | None = None,
                 pad_value: int = -1):
    """Returns (block_table [B][max_blocks] int32, num_blocks).

    Sequence b owns ceil(L_b / P) blocks; ids come from one seeded permutation of
    the pool, dealt out in sequence order. Unused table entries hold pad_value.
    """
    need = blocks_needed(lens, P)
    total = sum(need) + spare_blocks
    mb = max(need + [1]) if max_blocks is None else max_blocks
    perm = torch.randperm(total, generator=generator("blocks", *parts)).to(torch.int32)
    bt = torch.full((len(need), mb), pad_value, dtype=torch.int32)
    k = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[k:k + n]
        k += n
    return bt, total


def slot_of(block_table: torch.Tensor, b: int, t: int, P: int) -> int:
    return int(block_table[b, t // P]) * P + t % P


def token_slots(block_table: torch.Tensor, lens, P: int, first=None, last=None) -> torch.Tensor:
    """Slots of tokens [first_b, last_b) of every sequence, concatenated in (b, t) order."""
    out = []
    for b, L in enumerate(lens):
        lo = 0 if first is None else int(first[b])
        hi = int(L) if last is None else int(last[b])
        t = torch.arange(lo, hi, dtype=torch.int64)
        out.append(block_table[b, (t // P)].to(torch.int64) * P + t % P)
    return torch.cat(out).to(torch.int32) if out else torch.zeros(0, dtype=torch.int32)


def page_lists(lens, P: int, k: int, *parts) -> torch.Tensor:
    """[B][k] int32: the page of the newest token, plus k-1 distinct earlier pages."""
    rows = []
    for b, L in enumerate(lens):
        last = (int(L) - 1) // P
        g = generator("pages", b, *parts)
        take = min(k - 1, last)
        earlier = torch.randperm(last, generator=g)[:take].sort().values if last > 0 else \
            torch.zeros(0, dtype=torch.int64)
        row = torch.cat([earlier, torch.tensor([last])]).to(torch.int32)
        if row.numel() < k:
            row = torch.cat([row, torch.full((k - row.numel(),), -1, dtype=torch.int32)])
        rows.append(row)
    return torch.stack(rows)


def raw_numpy(t: torch.Tensor):
    """Raw element bits of a CPU tensor as numpy: uint16 for 2-byte types, float32 for fp32."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view("uint16")


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one benchmarked decode workload."""
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    dtype: str
    block_size: int
    layers: int = 1
    ctx_lo: int = 0
    ctx_hi: int = 0
    steps: int = 1
    window: int = 0
    sinks: int = 0
    window_layers: tuple = ()
    pages_per_step: int = 0

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    def kv_bytes_per_token(self) -> int:
        return 2 * self.kv_heads * self.head_dim * DTYPE_BYTES[self.dtype]


# The five decode workloads (shapes of the models and serving setups the pages discuss).
WORKLOADS = {
    "tiny_mha_f32": Workload("tiny_mha_f32", 1, 8, 8, 64, "f32", 16, ctx_lo=256, ctx_hi=256),
    "llama3_8b_layer_bf16": Workload("llama3_8b_layer_bf16", 32, 32, 8, 128, "bf16", 16,
                                     ctx_lo=1024, ctx_hi=4096),
    "qwen25_1p5b_28l_bf16": Workload("qwen25_1p5b_28l_bf16", 64, 12, 2, 128, "bf16", 16,
                                     layers=28, ctx_lo=4096, ctx_hi=4096, steps=32),
    "llama3_8b_kvsparse_bf16": Workload("llama3_8b_kvsparse_bf16", 8, 32, 8, 128, "bf16", 16,
                                        layers=32, ctx_lo=7000, ctx_hi=30000, window=512,
                                        sinks=4, window_layers=tuple(range(8, 24))),
    "mha7b_pagesel_f16": Workload("mha7b_pagesel_f16", 16, 32, 32, 128, "f16", 32,
                                  ctx_lo=32768, ctx_hi=32768, pages_per_step=16),
}


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)
