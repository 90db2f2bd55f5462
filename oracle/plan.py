"""Oracle for the RaggedShard communication-buffer layout (test infrastructure).

Only tests, the smoke check and the benchmark's CPU baseline use this module;
the product never does.

Problem (veScale-FSDP: Flexible and High-Performance FSDP at Scale, section
"Planning Algorithm", the formulation under Figure 6): a group T of tensors is
laid out in one flat buffer split into m equal shards of S elements; rank k
owns [k*S, (k+1)*S).  Tensor t occupies [l_t, r_t).  Minimise S subject to

  * non-split blocks: a shard boundary k*S that falls strictly inside
    [l_t, r_t) must fall a whole number of granules g_t after l_t;
  * contiguous tensor memory: r_t - l_t equals the tensor's element count
    and tensors do not overlap (padding goes between tensors, never inside
    one, as in Figure 6(b));
  * balanced load: every rank holds exactly S elements (tail padding), the
    equal-size rule of the FlatParameter section of "PyTorch FSDP:
    Experiences on Scaling Fully Sharded Data Parallel".

Readings used here (the pages are garbled or silent on these):
  * tensor order is kept as given (the pages adopt the default order);
  * an extra alignment A: S and every l_t are multiples of A (A=1 is the
    pure problem);
  * among the layouts with minimal S, the one with the lexicographically
    smallest offsets is chosen (greedy earliest placement).

The pages' own solver is a DP heuristic whose text is not given; this oracle
solves the fixed-order problem exactly instead: scan S upward from a lower
bound, and for each S place tensors greedily at their earliest valid offset.
Greedy is exact for a fixed S: whether an offset is valid for a tensor does
not depend on the other tensors, so ending each tensor as early as possible
can only widen the choices of the next one.  Feasibility is not monotone in
S, which is why S is scanned instead of bisected.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple


@dataclass(frozen=True)
class Item:
    """A tensor as the planner sees it: element count E and granule g."""

    numel: int
    granule: int


def items_from_specs(specs) -> List[Item]:
    """Map row-major tensor specs to (E, g): g = gran_rows * cols, or 1."""
    out = []
    for s in specs:
        e = s.rows * s.cols
        g = s.gran_rows * s.cols if s.gran_rows > 0 else 1
        out.append(Item(e, g))
    return out


def round_up(x: int, a: int) -> int:
    return -(-x // a) * a


def inner_boundaries(l: int, e: int, S: int, m: int) -> List[int]:
    """Shard boundaries k*S (1 <= k <= m-1) strictly inside (l, l+e)."""
    return [k * S for k in range(1, m) if l < k * S < l + e]


def offset_is_valid(l: int, it: Item, S: int, m: int, A: int) -> bool:
    """The per-tensor constraints for a tensor placed at offset l."""
    if l < 0 or l % A != 0 or l + it.numel > m * S:
        return False
    return all((b - l) % it.granule == 0 for b in inner_boundaries(l, it.numel, S, m))


def earliest_offset(lo: int, it: Item, S: int, m: int, A: int) -> Optional[int]:
    """Smallest valid offset >= lo, or None.

    Walks candidate offsets upward.  When the first inner boundary b is not a
    whole number of granules away, no offset before the next one that is
    (b - l' divisible by lcm(g, A)) can be valid, because b stays inside the
    tensor while l' < b.  When b is aligned but a later inner boundary is
    not, every offset below b keeps that later boundary inside and misaligned
    (their distance changes by multiples of g only), so the walk moves to b.
    """
    L = it.granule * A // math.gcd(it.granule, A)
    l = round_up(lo, A)
    while l + it.numel <= m * S:
        inner = inner_boundaries(l, it.numel, S, m)
        bad = [b for b in inner if (b - l) % it.granule != 0]
        if not bad:
            return l
        b = inner[0]
        if (b - l) % it.granule != 0:
            # next offset in (l, b) aligned to b, else b itself
            steps = (b - l - 1) // L
            cand = b - steps * L
            l = cand if l < cand < b else b
        else:
            l = b
    return None


def greedy_offsets(items: Sequence[Item], m: int, S: int, A: int) -> Optional[List[int]]:
    if S % A != 0:
        return None
    offs = []
    end = 0
    for it in items:
        l = earliest_offset(end, it, S, m, A)
        if l is None:
            return None
        offs.append(l)
        end = l + it.numel
    return offs


def lower_bound(items: Sequence[Item], m: int, A: int) -> int:
    """max(ceil(E/m), max_t min(g_t, E_t)) rounded up to A.

    No block can be cut, so a shard is at least as large as every tensor's
    first (possibly partial) block.
    """
    total = sum(it.numel for it in items)
    lb = max([-(-total // m)] + [min(it.granule, it.numel) for it in items])
    return round_up(max(lb, 1), A)


def shard_multiple_required(items: Sequence[Item], S: int) -> bool:
    """Necessary condition: a tensor longer than 2S has two inner boundaries
    S apart, both a whole number of granules from its start, so S must be a
    multiple of its granule."""
    return all(S % it.granule == 0 for it in items if it.numel > 2 * S)


@dataclass
class Plan:
    S: int
    offsets: List[int]
    m: int
    total: int  # m * S

    @property
    def numel(self) -> int:
        return self.total


def plan(items: Sequence[Item], m: int, A: int = 1, S_cap: int = 0) -> Optional[Plan]:
    """Minimum-S layout with tensor order kept (greedy earliest offsets)."""
    S = lower_bound(items, m, A)
    total = sum(it.numel for it in items)
    # every tensor fits in shard 0 once S covers all of them back to back
    cap = S_cap if S_cap > 0 else round_up(total, A) + len(items) * A
    while S <= cap:
        if shard_multiple_required(items, S):
            offs = greedy_offsets(items, m, S, A)
            if offs is not None:
                return Plan(S, offs, m, m * S)
        S += A
    return None


def plan_bruteforce(items: Sequence[Item], m: int, A: int = 1) -> Optional[Tuple[int, List[int]]]:
    """Exhaustive search for tiny inputs: for S = A, 2A, ... enumerate every
    offset vector whose entries are individually valid and in order, and
    return the first S with any layout and its lexicographically smallest
    offsets."""
    total = sum(it.numel for it in items)
    for S in range(A, round_up(total, A) + len(items) * A + 1, A):
        per = [[l for l in range(0, m * S + 1, A) if offset_is_valid(l, it, S, m, A)]
               for it in items]
        best = None

        def rec(t: int, end: int, acc: List[int]):
            nonlocal best
            if best is not None:
                return
            if t == len(items):
                best = list(acc)
                return
            for l in per[t]:
                if l >= end:
                    acc.append(l)
                    rec(t + 1, l + items[t].numel, acc)
                    acc.pop()
                    if best is not None:
                        return

        rec(0, 0, [])
        if best is not None:
            return S, best
    return None


def check_layout(items: Sequence[Item], starts: Sequence[int], ends: Sequence[int],
                 bounds: Sequence[int], A: int = 1) -> List[str]:
    """List the constraint violations of an explicit layout.

    starts/ends: per-tensor [l_t, r_t); bounds: m+1 rank boundaries
    b_0=0 < ... < b_m.  Reports the three failure modes of naive
    concatenation (Figure 6(a)): a block cut by a rank boundary, a tensor
    whose memory is not contiguous, and unequal per-rank sizes.
    """
    errs = []
    sizes = [bounds[k + 1] - bounds[k] for k in range(len(bounds) - 1)]
    if len(set(sizes)) != 1:
        errs.append("imbalanced load: rank sizes %s" % sizes)
    for t, it in enumerate(items):
        l, r = starts[t], ends[t]
        if r - l != it.numel:
            errs.append(f"tensor {t}: non-contiguous memory ({r - l} slots for {it.numel})")
        if l % A:
            errs.append(f"tensor {t}: offset {l} not a multiple of {A}")
        if t and l < ends[t - 1]:
            errs.append(f"tensor {t}: overlaps tensor {t - 1}")
        for b in bounds[1:-1]:
            if l < b < r and (b - l) % it.granule:
                errs.append(f"tensor {t}: block split by boundary {b}")
    if ends and ends[-1] > bounds[-1]:
        errs.append("last tensor ends past the buffer")
    return errs


def fragments(items: Sequence[Item], offsets: Sequence[int], S: int, m: int):
    """(tensor, rank, buffer_lo, buffer_hi) for every non-empty tensor/rank
    intersection, in buffer order."""
    out = []
    for t, (it, l) in enumerate(zip(items, offsets)):
        r = l + it.numel
        for k in range(l // S, min(m, (r - 1) // S + 1)):
            lo, hi = max(l, k * S), min(r, (k + 1) * S)
            if lo < hi:
                out.append((t, k, lo, hi))
    return out


def peak_param_bytes(S: int, m: int, k_full: int = 4, k_low: int = 2) -> int:
    """Per-rank parameter memory of one unit with native mixed precision:
    the sharded full-precision copy plus the unsharded low-precision copy,
    K_full * psi / F + K_low * psi with psi = m * S and F = m ("PyTorch FSDP",
    FlatParameter and native mixed precision sections)."""
    psi = m * S
    return k_full * psi // m + k_low * psi


def padding_fraction(items: Sequence[Item], S: int, m: int) -> float:
    total = sum(it.numel for it in items)
    return (m * S - total) / total


# ---------------------------------------------------------------- orders
#
# The pages compare three tensor orders for the planner - the given one, one
# by block size and one by tensor shape - and keep the given one, which was
# optimal or near it in their runs (veScale-FSDP, "Planning Algorithm").
# They do not define the other two; the readings here are: by block size =
# granule elements descending, by shape = (rows, cols) descending, both
# stable (equal keys keep the given order).  "best" plans all three and
# keeps the smallest S, ties going to the earlier of given, block, shape.

ORDER_KINDS = ("given", "block", "shape")


def order_perm(specs, kind: str) -> List[int]:
    """Buffer order: perm[i] is the index of the tensor placed i-th."""
    idx = list(range(len(specs)))
    if kind == "given":
        return idx
    if kind == "block":
        gran = [s.gran_rows * s.cols if s.gran_rows > 0 else 1 for s in specs]
        return sorted(idx, key=lambda t: gran[t], reverse=True)
    if kind == "shape":
        return sorted(idx, key=lambda t: (specs[t].rows, specs[t].cols), reverse=True)
    raise ValueError(kind)


def plan_ordered(specs, m: int, A: int = 1, kind: str = "given"):
    """-> (perm, offsets indexed as specs, S) or None.  The plan of the
    tensors taken in buffer order perm; kind "best" tries the three orders."""
    kinds = ORDER_KINDS if kind == "best" else (kind,)
    best = None
    for k in kinds:
        perm = order_perm(specs, k)
        items = items_from_specs([specs[t] for t in perm])
        p = plan(items, m, A)
        if p is None:
            continue
        if best is None or p.S < best[2]:
            offs = [0] * len(specs)
            for i, t in enumerate(perm):
                offs[t] = p.offsets[i]
            best = (perm, offs, p.S)
    return best
