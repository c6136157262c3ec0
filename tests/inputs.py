"""Seeded synthetic inputs for the QSA decode path.

This module only draws random numbers and lays them out: it holds none of the
method's arithmetic (no pooling, scoring, selection or attention).  Both the
CPU oracle and the HIP path take their inputs from here, so neither ever
feeds the other.

Workload shapes follow the model-free F32 checkpoint sizes the notes report
(AFN-016 "A sparse mask is not sparse attention", §What the checkpoint
measures: 65,537, 100,000 and 262,144 visible tokens; AFN-017 "Top-k chooses
the set; time chooses the order", capsule evidence: the dense-parity sweep at
0-5 and 2,047-2,052 tokens).  Draw order is fixed: index queries, raw index
keys, attention queries, K, V, slot map.

Every tensor is produced with torch.Generator on the requested device, so a
config drawn on the GPU is copied to the host for the oracle (and a config
drawn on the CPU is copied to the GPU for the HIP path).
"""
from dataclasses import dataclass, field
from typing import List, Optional

import torch

GROUP = 4
BUDGET = 512


@dataclass
class Spec:
    name: str
    seq_lens: List[int]            # tokens per sequence (the last query sees all of them)
    queries: int = 1               # causal query rows per sequence (1 = decode)
    h_i: int = 4                   # indexer heads
    d_i: int = 32                  # indexer head dim
    h_q: int = 1                   # attention query heads
    h_kv: int = 1                  # attention KV heads
    d: int = 64                    # attention head dim
    budget: int = BUDGET           # groups kept per row
    keys: str = "normal"           # "normal" | "grid" | "grid_dup" | "zero_query"
    slots: str = "identity"        # "identity" | "ring" | "perm" | "shared_perm"
    capacity: Optional[int] = None  # ring capacity
    extra: dict = field(default_factory=dict)

    @property
    def batch(self):
        return len(self.seq_lens)

    @property
    def rows(self):
        return self.batch * self.queries


def spec(name: str, seed: int = 1) -> Spec:
    """The five named workloads:
      tail_2055         one row of 2,055 tokens (513 groups + 3 tail), grid keys
      ring_65537        one row of 65,537 tokens, ring slot map of capacity 70,000
      dup_100000        one row of 100,000 tokens, 20% duplicated groups (ties)
      decode_32x262144  decode batch of 32 rows of 262,144 tokens, shared
                        8,388,608-slot cache
      chunk_8x256       8 sequences of 2,051..262,144 tokens, 256 causal queries
    """
    if name == "tail_2055":
        return Spec("tail_2055", [2055], h_i=4, d_i=32, h_q=1, h_kv=1, d=64, keys="grid",
                    slots="identity")
    if name == "ring_65537":
        return Spec("ring_65537", [65537], h_i=8, d_i=64, h_q=1, h_kv=1, d=128, keys="normal",
                    slots="ring", capacity=70000)
    if name == "dup_100000":
        return Spec("dup_100000", [100000], h_i=8, d_i=64, h_q=8, h_kv=1, d=128, keys="grid_dup",
                    slots="perm")
    if name == "decode_32x262144":
        return Spec("decode_32x262144", [262144] * 32, h_i=16, d_i=128, h_q=32, h_kv=4, d=128,
                    keys="normal", slots="shared_perm")
    if name == "chunk_8x256":
        g = torch.Generator().manual_seed(1000 + seed)
        lens = torch.randint(2051, 262145, (8,), generator=g).tolist()
        return Spec("chunk_8x256", lens, queries=256, h_i=16, d_i=128, h_q=32, h_kv=4, d=128,
                    keys="normal", slots="identity")
    raise KeyError(name)


def _grid(shape, gen, device):
    # uniform on {-2,-1,0,1,2}/8: products and short sums are exact in F32
    return torch.randint(-2, 3, shape, generator=gen, device=device,
                         dtype=torch.int32).to(torch.float32) / 8.0


def make(s: Spec, seed: int = 1, device="cpu", kv_poison_nan: bool = True) -> dict:
    """Draw every input of spec s.

    Returns a dict of tensors on `device`:
      index_q  [rows][h_i][d_i] f32     raw_keys [T][d_i] f32 (all sequences, flat)
      raw_off  [batch] int64 token offset of each sequence in raw_keys / slot_map
      q        [rows][h_q][d] f32       k_cache, v_cache [S][h_kv][d] f32
      slot_map [T] int32                seq_len [batch] int32
    plus the python ints kv_slots, total_tokens and the spec.
    Row r = b*queries + j sees seq_len[b] - queries + 1 + j tokens.
    """
    dev = torch.device(device)
    gen = torch.Generator(device=dev).manual_seed(seed)
    lens = list(s.seq_lens)
    total = int(sum(lens))
    rows = s.rows
    off = [0]
    for n in lens[:-1]:
        off.append(off[-1] + n)

    # 1. index queries
    if s.keys in ("grid", "grid_dup"):
        index_q = _grid((rows, s.h_i, s.d_i), gen, dev)
    elif s.keys == "zero_query":
        index_q = torch.zeros((rows, s.h_i, s.d_i), device=dev)
        torch.randn((1,), generator=gen, device=dev)  # keep the draw sequence aligned
    else:
        index_q = torch.randn((rows, s.h_i, s.d_i), generator=gen, device=dev)

    # 2. raw index keys
    if s.keys in ("grid", "grid_dup"):
        raw = _grid((total, s.d_i), gen, dev)
    else:
        raw = torch.randn((total, s.d_i), generator=gen, device=dev)
    if s.keys == "grid_dup":
        # 20% of each sequence's complete groups become exact copies of another
        # (not copied-over) group's four raw keys, so pooled keys tie exactly
        for b, n in enumerate(lens):
            g = n // GROUP
            n_dup = g // 5
            if n_dup == 0 or g - n_dup == 0:
                continue
            perm = torch.randperm(g, generator=gen, device=dev)
            dst, keep = perm[:n_dup], perm[n_dup:]
            src = keep[torch.randint(0, keep.numel(), (n_dup,), generator=gen, device=dev)]
            view = raw[off[b]:off[b] + g * GROUP].view(g, GROUP, s.d_i)
            view[dst] = view[src]

    # 3. attention queries
    q = torch.randn((rows, s.h_q, s.d), generator=gen, device=dev)

    # 6 (drawn after K/V below). slot-map layout decides the cache size
    if s.slots == "identity":
        kv_slots = total
    elif s.slots == "ring":
        assert s.batch == 1
        kv_slots = int(s.capacity)
    elif s.slots == "perm":
        kv_slots = total
    elif s.slots == "shared_perm":
        kv_slots = total
    else:
        raise KeyError(s.slots)

    # 4-5. K and V caches
    k_cache = torch.randn((kv_slots, s.h_kv, s.d), generator=gen, device=dev)
    v_cache = torch.randn((kv_slots, s.h_kv, s.d), generator=gen, device=dev)

    # 6. slot map, logical token -> physical cache slot
    if s.slots == "identity":
        slot_map = torch.arange(total, device=dev, dtype=torch.int32)
    elif s.slots == "ring":
        offset = int(torch.randint(0, kv_slots, (1,), generator=gen, device=dev).item())
        slot_map = ((torch.arange(total, device=dev, dtype=torch.int64) + offset)
                    % kv_slots).to(torch.int32)
        if kv_poison_nan and kv_slots > total:
            # slots the ring never maps hold NaN: reading one would show up
            mapped = torch.zeros(kv_slots, dtype=torch.bool, device=dev)
            mapped[slot_map.long()] = True
            k_cache[~mapped] = float("nan")
            v_cache[~mapped] = float("nan")
    elif s.slots == "perm":
        slot_map = torch.cat([
            torch.randperm(n, generator=gen, device=dev).to(torch.int32) + o
            for n, o in zip(lens, off)])
    else:  # shared_perm: one permutation of the pool split into disjoint chunks
        slot_map = torch.randperm(kv_slots, generator=gen, device=dev).to(torch.int32)

    return dict(
        spec=s,
        index_q=index_q.contiguous(),
        raw_keys=raw.contiguous(),
        raw_off=torch.tensor(off, dtype=torch.int64, device=dev),
        q=q.contiguous(),
        k_cache=k_cache.contiguous(),
        v_cache=v_cache.contiguous(),
        slot_map=slot_map.contiguous(),
        seq_len=torch.tensor(lens, dtype=torch.int32, device=dev),
        kv_slots=kv_slots,
        total_tokens=total,
    )


def custom(name, seq_lens, **kw) -> Spec:
    """A free-form spec for edge-case and ragged tests."""
    return Spec(name, list(seq_lens), **kw)


def row_tokens(s: Spec, row: int) -> int:
    """Visible tokens of a row: seq_len[b] - queries + 1 + j for row b*queries + j."""
    b, j = divmod(row, s.queries)
    return s.seq_lens[b] - s.queries + 1 + j


def sweep_prefixes():
    """Dense-parity sweep points (AFN-017 capsule evidence)."""
    return [0, 1, 2, 3, 4, 5, 2047, 2048, 2049, 2050, 2051, 2052]
