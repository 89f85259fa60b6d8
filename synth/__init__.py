"""Seeded synthetic inputs for packed QSA decode.

This module only draws random numbers and lays them out: it holds none of
the decode's arithmetic and none of the quantizers.  Both the tests (oracle
side and GPU side) and the benchmark take their inputs from here.

Shapes follow the packed decode contract of the page "fix(qsa): restore
SM121 correctness with Humanize and Kernel Design Agent" (section
"Changes"): one bf16 query row per packed sequence, head dim 256, 24 Q heads
over 2 KV heads (TP1) or 12 over 1 (TP2), up to 2055 selected pool slots per
row, indices packed with cu_seqlens.  Index lists keep their drawn order and
may repeat a slot.

Random source: numpy ``default_rng(seed)`` (PCG64).  Floats are drawn as
float32 and rounded to bf16 by torch on the CPU (round to nearest even).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 256
GQA = 12
CAPACITY = 2055


@dataclass
class QsaCase:
    """One decode call's inputs on the host (torch CPU tensors)."""
    q: "object"            # [bs, hq, 256] bf16
    k_pool: "object"       # [slots, hkv, 256] bf16
    v_pool: "object"       # [slots, hkv, 256] bf16
    sel: np.ndarray        # [n_sel] int32
    cu: np.ndarray         # [bs + 1] int32
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def bs(self) -> int:
        return int(self.cu.shape[0] - 1)

    @property
    def hkv(self) -> int:
        return int(self.k_pool.shape[1])

    @property
    def hq(self) -> int:
        return int(self.q.shape[1])

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.cu)


def to_bf16(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return to_bf16(x)


def pack(lists) -> tuple[np.ndarray, np.ndarray]:
    """List of per-row index arrays -> (sel, cu_seqlens)."""
    lens = np.array([len(x) for x in lists], dtype=np.int64)
    cu = np.zeros(len(lists) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    sel = (np.concatenate([np.asarray(x, dtype=np.int32) for x in lists])
           if len(lists) and lens.sum() else np.zeros(0, dtype=np.int32))
    return np.ascontiguousarray(sel, dtype=np.int32), cu


def draw_indices(rng: np.random.Generator, length: int, slots: int,
                 dup_prob: float = 0.0, run: tuple[int, int] = (2, 8)) -> np.ndarray:
    """Uniform slot ids with replacement, in drawn order.  With probability
    ``dup_prob`` an entry starts a run that repeats the previous id so that it
    appears run[0]..run[1] times in a row."""
    idx = rng.integers(0, slots, size=length, dtype=np.int64).astype(np.int32)
    if dup_prob > 0 and length > 1:
        starts = rng.random(length) < dup_prob
        runs = rng.integers(run[0], run[1] + 1, size=length)
        i = 1
        while i < length:
            if starts[i]:
                r = int(runs[i]) - 1          # extra copies of the previous id
                end = min(length, i + r)
                idx[i:end] = idx[i - 1]
                i = end
            else:
                i += 1
    return idx


def make_case(*, lengths, slots: int, hkv: int, seed: int, dup_prob: float = 0.0,
              peaked_frac: float = 0.0, peaked_mult: float = 8.0,
              name: str = "") -> QsaCase:
    """Generic case: q, K, V ~ N(0, 1) in bf16; per-row uniform indices."""
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in lengths]
    bs = len(lengths)
    hq = GQA * hkv
    q = normal_bf16(rng, (bs, hq, HEAD_DIM))
    k = normal_bf16(rng, (slots, hkv, HEAD_DIM))
    v = normal_bf16(rng, (slots, hkv, HEAD_DIM))
    if peaked_frac > 0:
        import torch
        mask = torch.from_numpy(rng.random((slots, hkv)) < peaked_frac)
        # x8 is a power of two, so the scaled rows stay exact in bf16
        k[mask] = k[mask] * peaked_mult
    lists = [draw_indices(rng, n, slots, dup_prob) for n in lengths]
    sel, cu = pack(lists)
    return QsaCase(q=q, k_pool=k, v_pool=v, sel=sel, cu=cu, name=name,
                   meta=dict(seed=seed, slots=slots, hkv=hkv))


# ---------------------------------------------------------------------------
# Named workloads.  Their recipes are stated in the design notes.
# ---------------------------------------------------------------------------

def case_bs1_tp1(seed: int = 101) -> QsaCase:
    """bs=1, 24Q/2KV, pools [4096, 2, 256], 128 uniform indices."""
    return make_case(lengths=[128], slots=4096, hkv=2, seed=seed, name="bs1_tp1_L128")


def mixed_lengths_bs16(rng: np.random.Generator) -> list[int]:
    """bs=16: 8 short rows L~U[1,64], 4 saturated (2055), 4 L~U[65,2054],
    row order shuffled."""
    short = rng.integers(1, 65, size=8)
    mid = rng.integers(65, CAPACITY, size=4)
    lens = np.concatenate([short, np.full(4, CAPACITY), mid])
    rng.shuffle(lens)
    return [int(x) for x in lens]


def case_bs16_tp2_mixed(seed: int = 102, slots: int = 65536) -> QsaCase:
    """bs=16, 12Q/1KV, pools [65536, 1, 256], mixed lengths, duplicates allowed."""
    lens = mixed_lengths_bs16(np.random.default_rng(seed ^ 0x5EED))
    return make_case(lengths=lens, slots=slots, hkv=1, seed=seed, name="bs16_tp2_mixed")


def case_bs128_tp1_saturated(seed: int = 103, slots: int = 262144, bs: int = 128,
                             hkv: int = 2) -> QsaCase:
    """bs=128, 24Q/2KV, pools [262144, 2, 256], all rows at 2055, 5% of the
    (slot, kv-head) key rows scaled x8 (peaked softmax).  bs and the KV head
    count can be changed for sweeps."""
    return make_case(lengths=[CAPACITY] * bs, slots=slots, hkv=hkv, seed=seed,
                     peaked_frac=0.05, name=f"bs{bs}_hkv{hkv}_sat2055_peaked")


def quant_lengths_bs64(rng: np.random.Generator, bs: int = 64) -> list[int]:
    return [int(x) for x in rng.integers(256, CAPACITY + 1, size=bs)]


def case_bs64_tp1_quantsrc(seed: int, slots: int = 131072, bs: int = 64) -> QsaCase:
    """bs=64, 24Q/2KV, bf16 source pools [131072, 2, 256] ~ N(0, 1) that the
    caller quantizes; lengths L~U[256, 2055]."""
    lens = quant_lengths_bs64(np.random.default_rng(seed ^ 0x5EED), bs)
    return make_case(lengths=lens, slots=slots, hkv=2, seed=seed,
                     name=f"bs{bs}_tp1_quantsrc")


SWEEP_BS = list(range(1, 17)) + [17, 24, 32, 48, 64, 96, 128]


def sweep_lengths(rng: np.random.Generator, bs: int, kind: str) -> list[int]:
    """Replay-sweep lengths: short L~U[1,32], medium L~U[960,1088],
    saturated L=2055."""
    if kind == "short":
        return [int(x) for x in rng.integers(1, 33, size=bs)]
    if kind == "medium":
        return [int(x) for x in rng.integers(960, 1089, size=bs)]
    if kind == "saturated":
        return [CAPACITY] * bs
    raise ValueError(kind)


def sweep_empty_rows(bank: int, bs: int) -> list[int]:
    """Rows a sweep bank leaves empty: none, except in every fourth bank
    (bank % 4 == 3), which empties row 7*bank mod bs and, from bs = 4, also
    the row half a batch further.  At bs = 1 such a bank is an all-empty
    call."""
    if bank % 4 != 3:
        return []
    rows = {(7 * bank) % bs}
    if bs >= 4:
        rows.add((7 * bank + bs // 2) % bs)
    return sorted(rows)


def sweep_bank(seed: int, bs: int, kind: str, slots: int, banks: int = 8,
               dup_prob: float = 0.1):
    """``banks`` different (sel, cu) packings for one sweep point, each with
    duplicate runs (probability 0.1 per entry, runs of 2..8), and with the
    zero-length rows of sweep_empty_rows (the lists are drawn first and then
    emptied, so the other rows keep their draws).  All banks are padded to
    the same sel length so they can be copied into one captured buffer."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(banks):
        lens = sweep_lengths(rng, bs, kind)
        lists = [draw_indices(rng, n, slots, dup_prob) for n in lens]
        for j in sweep_empty_rows(i, bs):
            lists[j] = lists[j][:0]
        out.append(pack(lists))
    cap = max(s.shape[0] for s, _ in out)
    padded = []
    for s, c in out:
        p = np.zeros(max(cap, 1), dtype=np.int32)
        p[: s.shape[0]] = s
        padded.append((p, c))
    return padded


def tiered_lists(rng: np.random.Generator, lengths, slots: int, recent: np.ndarray,
                 hot_frac: float, dup_prob: float = 0.0) -> tuple[np.ndarray, np.ndarray]:
    """Packed lists for a tiered pool: each entry is, with probability
    ``hot_frac``, a uniform draw from ``recent`` (the most recently written
    slot ids) and otherwise a uniform draw from all slots; duplicate runs as
    in draw_indices."""
    lists = []
    recent = np.asarray(recent, dtype=np.int64)
    for n in lengths:
        idx = draw_indices(rng, int(n), slots, dup_prob).astype(np.int64)
        pick = rng.random(int(n)) < hot_frac
        idx[pick] = recent[rng.integers(0, len(recent), size=int(pick.sum()))]
        lists.append(idx.astype(np.int32))
    return pack(lists)


def write_batches(rng: np.random.Generator, order: np.ndarray, batches: int) -> list[np.ndarray]:
    """Split a write order of slot ids into ``batches`` consecutive calls of
    random sizes."""
    n = len(order)
    if batches <= 1 or n < 2:
        return [np.asarray(order)]
    cuts = np.sort(rng.choice(np.arange(1, n), size=min(batches - 1, n - 1), replace=False))
    return np.split(np.asarray(order), cuts)


def index_inputs(rng: np.random.Generator, ctx, *, hi: int = 4, di: int = 64, c: int = 4,
                 max_tokens: int | None = None, weights: bool = True, slots: int = 1 << 20):
    """Inputs of the indexer step for rows of context lengths ``ctx``: index
    query heads q [bs, hi, di] and one compressed key per block row of a
    key pool [bs * max_blocks, di] (bf16 N(0, 1)); a block table that
    scatters each row's blocks over the pool (a random permutation); a
    token -> KV slot table per row (distinct slots drawn from [0, slots));
    head weights U[0.5, 1.5) or None."""
    bs = len(ctx)
    max_tokens = max_tokens or max(max(int(t) for t in ctx), 1)
    max_blocks = max_tokens // c + 1
    n_kpool = bs * max_blocks
    q = normal_bf16(rng, (bs, hi, di))
    k = normal_bf16(rng, (n_kpool, di))
    bt = rng.permutation(n_kpool).reshape(bs, max_blocks).astype(np.int32)
    r2t = np.stack([rng.choice(slots, size=max_tokens, replace=False) for _ in range(bs)])
    w = (rng.random((bs, hi), dtype=np.float32) + np.float32(0.5)) if weights else None
    return dict(q=q, k_pool=k, block_table=bt, req_to_token=r2t.astype(np.int32),
                ctx_len=np.asarray(ctx, np.int32), weights=w)

