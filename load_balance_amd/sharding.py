"""Context-parallel sharding of a packed sequence, and one rank's sharded ring on one GPU.

Which query tokens each of cp ranks holds:

* ``zigzag``: the pack is cut into 2*cp equal chunks and rank i holds chunks i
  and 2*cp-1-i ("03 · 长文负载均衡", section 4.2).  On a packed sequence this
  balances the ranks only in expectation (same page, section 1.2; the
  131072-token pack of seed 0 at cp = 8 leaves the busiest rank 1.63x the mean).
* ``per_document``: every document is cut into 2*cp chunks and rank i takes
  chunks i and 2*cp-1-i of each; a length that is not a multiple of 2*cp leaves
  a tail of len mod 2*cp tokens, dealt round-robin with one pointer over the
  whole pack (section 4.3, WLB-LLM): every rank gets the same causal area of
  every document and the same token count to within one.
* ``striped``: stripes of ``width`` tokens dealt to ranks in turn (section 4.2,
  Striped Attention).
* ``dispatch``: MagiAttention's dispatch solver (section 4.4): the pack is cut
  into ``n_chunks`` equal chunks along the query axis; each chunk's mask area
  (its visible (query, key) pairs) is computed, and the chunks are dealt, largest
  area first, each to the least-loaded rank that holds fewer than n_chunks / cp
  chunks (a min-heap).  Token counts stay equal (the linear term of the cost) while
  the greedy evens the area (the quadratic term).  On one causal document with
  n_chunks = 2*cp it gives exactly the zigzag pairing.

At ring step t a rank attends its queries to the keys and values of rank
(r - t) mod cp ("长序列训练与上下文并行", Ring Attention) and folds the step's
partial result into its running one with ``lse_merge``.  Every step is one
``block_attn_fwd`` (positions and document ids travel with the tokens, so any
token set works) -- planned up front with ``plan_block_steps``, since a step's
metadata is known before its keys and values arrive.

Per-document sharding trades balance for shorter runs, and a short query run
still costs a whole tile (section 3.3; section 4.3 on WLB-LLM's adaptive choice
between per-sequence and per-document sharding by predicted latency with
tile-rounded cost).  ``predicted_work`` counts the key blocks and work items the
attention kernel would run for a rank; a linear time model over blocks, items
and ring steps, with coefficients fitted to measured rank times ("数据并行负载均衡",
section 4.3: costs from a fitted model; "03 · 长文负载均衡", section 2.2:
coefficients fitted by offline profiling), turns them into a predicted time,
and ``choose_sharding`` picks the rule whose busiest rank is predicted fastest.
"""
from __future__ import annotations

import heapq

import numpy as np
import torch

BLOCK_KEYS = 64  # keys per block of the attention kernel (LB_BLOCK_KEYS)
FUSED_TILE_CAP = 4096  # query tiles one fused ring takes (lb_plan_ring_fused)


# --------------------------------------------------------------------------
# sharding rules: per rank, ascending global token indices
# --------------------------------------------------------------------------
def zigzag_tokens(total: int, cp: int):
    if total % (2 * cp):
        raise ValueError("zigzag sharding needs a pack length divisible by 2*cp")
    c = total // (2 * cp)
    return [np.r_[i * c:(i + 1) * c, (2 * cp - 1 - i) * c:(2 * cp - i) * c].astype(np.int64) for i in range(cp)]


def per_document_tokens(lengths, cp: int):
    parts = [[] for _ in range(cp)]
    start, deal = 0, 0
    for n in (int(x) for x in lengths):
        c = n // (2 * cp)
        for i in range(cp):
            parts[i].append(np.arange(start + i * c, start + (i + 1) * c))
            parts[i].append(np.arange(start + (2 * cp - 1 - i) * c, start + (2 * cp - i) * c))
        tail = np.arange(start + 2 * cp * c, start + n)
        owner = (deal + np.arange(len(tail))) % cp
        for i in range(cp):
            parts[i].append(tail[owner == i])
        deal = (deal + len(tail)) % cp
        start += n
    return [np.sort(np.concatenate(p)).astype(np.int64) for p in parts]


def striped_tokens(total: int, cp: int, width: int = 1):
    t = np.arange(total, dtype=np.int64)
    return [t[(t // width) % cp == r] for r in range(cp)]


def chunk_areas(lengths, n_chunks: int) -> np.ndarray:
    """Per-document causal mask area of each of ``n_chunks`` equal query chunks: a token at
    position p of its document sees p + 1 keys."""
    lengths = np.asarray(lengths, dtype=np.int64)
    total = int(lengths.sum())
    if n_chunks <= 0 or total % n_chunks:
        raise ValueError("dispatch needs a pack length divisible by the chunk count")
    starts = np.repeat(np.cumsum(lengths) - lengths, lengths)
    seen = np.arange(total, dtype=np.int64) - starts + 1
    return seen.reshape(n_chunks, -1).sum(axis=1)


def dispatch_chunks(areas, cp: int):
    """Greedy dispatch of chunks to cp ranks of equal chunk counts: largest area first
    (ties: lower chunk id), each to the open rank with the least area (ties: lower rank),
    through a min-heap of (area, rank) that drops a rank once it is full."""
    n = len(areas)
    if n % cp:
        raise ValueError("dispatch needs a chunk count divisible by cp")
    capacity = n // cp
    heap = [(0, r) for r in range(cp)]
    held = [[] for _ in range(cp)]
    for c in sorted(range(n), key=lambda c: (-int(areas[c]), c)):
        load, r = heapq.heappop(heap)
        held[r].append(c)
        if len(held[r]) < capacity:
            heapq.heappush(heap, (load + int(areas[c]), r))
    return [sorted(h) for h in held]


def dispatch_tokens(lengths, cp: int, n_chunks: int):
    total = int(np.sum(lengths))
    size = total // n_chunks
    held = dispatch_chunks(chunk_areas(lengths, n_chunks), cp)
    return [np.concatenate([np.arange(c * size, (c + 1) * size) for c in h]).astype(np.int64) for h in held]


def shard_tokens(rule: str, lengths, cp: int, width: int = 1, n_chunks: int = 0):
    """Token sets of every rank under ``rule``; ``n_chunks`` (dispatch) defaults to 2*cp."""
    total = int(np.sum(lengths))
    if rule == "zigzag":
        return zigzag_tokens(total, cp)
    if rule == "per_document":
        return per_document_tokens(lengths, cp)
    if rule == "striped":
        return striped_tokens(total, cp, width)
    if rule == "dispatch":
        return dispatch_tokens(lengths, cp, n_chunks or 2 * cp)
    raise ValueError(f"unknown sharding rule {rule!r}")


def ring_source(rank: int, step: int, cp: int) -> int:
    return (rank - step) % cp


def token_meta(lengths):
    """Global position and document id (int32) of every token of a pack."""
    lengths = np.asarray(lengths, dtype=np.int64)
    pos = np.arange(int(lengths.sum()), dtype=np.int32)
    doc = np.repeat(np.arange(len(lengths), dtype=np.int32), lengths)
    return pos, doc


# --------------------------------------------------------------------------
# cost of a sharding: key blocks the attention kernel sweeps (host side)
# --------------------------------------------------------------------------
def _runs(pos, doc):
    """(start, length, first position, doc) of each run of equal doc and consecutive position."""
    if len(pos) == 0:
        return np.zeros((0, 4), dtype=np.int64)
    brk = np.flatnonzero((np.diff(doc) != 0) | (np.diff(pos) != 1)) + 1
    starts = np.r_[0, brk]
    lens = np.diff(np.r_[starts, len(pos)])
    return np.stack([starts, lens, pos[starts], doc[starts]], axis=1).astype(np.int64)


def predicted_work(q_pos, q_doc, kv_pos, kv_doc, tile_rows: int, shared_doc: int = -1):
    """(key blocks, work items) of one kv head for a query shard against a key/value shard:
    each run of the query shard is cut into tiles of ``tile_rows``; a tile sweeps, of every
    key run of its document, the blocks holding keys its last row can see, and is a work
    item when it sweeps any.  With a shared document (shared_doc >= 0), a run of any other
    document also sweeps every block of that document's key runs, runs next to each other in
    the key buffer taken as one span (as the planner does)."""
    qr, kr = _runs(np.asarray(q_pos), np.asarray(q_doc)), _runs(np.asarray(kv_pos), np.asarray(kv_doc))
    blocks = items = 0
    by_doc = {}
    far = -(1 << 30)  # a shared key run lies below every row
    for (_, ln, p0, d) in kr:
        by_doc.setdefault(int(d), []).append((int(ln), int(p0)))
    shared = [(kl, far) for kl in _full_spans(kr, shared_doc)]
    for (_, ln, p0, d) in qr:
        spans = list(by_doc.get(int(d), []))
        if shared_doc >= 0 and int(d) != shared_doc:
            spans += shared
        if not spans:
            continue
        last = p0 + np.minimum(np.arange(tile_rows, int(ln) + tile_rows, tile_rows), ln) - 1  # last row of each tile
        per_tile = np.zeros(len(last), dtype=np.int64)
        for (kl, kp0) in spans:
            keep = np.clip(last - kp0 + 1, 0, kl)
            per_tile += (keep + BLOCK_KEYS - 1) // BLOCK_KEYS
        blocks += int(per_tile.sum())
        items += int(np.count_nonzero(per_tile))
    return blocks, items


def _full_spans(runs, doc):
    """Lengths of the FULL spans that runs of ``doc`` make: runs next to each other in the
    buffer join into one span (every pair of a FULL span is seen, so positions play no part)."""
    out, end = [], -1
    for (st, ln, _, d) in runs:
        if doc < 0 or int(d) != doc:
            continue
        if out and end == st:
            out[-1] += int(ln)
        else:
            out.append(int(ln))
        end = int(st) + int(ln)
    return out


MAX_SPANS = 4  # spans one query run (or, in the backward, one key run) may meet (LB_MAX_SPANS)


def max_spans(lengths, tokens, shared_doc: int = -1) -> int:
    """The most spans any run of any rank meets on any ring step: the planner refuses a step
    where this exceeds MAX_SPANS.  A query run's spans are the key runs of its own document
    not wholly after it, plus, with a shared document, that document's FULL spans; in the
    backward's key-tile plan a key run of the shared document also meets the other documents'
    query runs as FULL spans."""
    pos, doc = token_meta(lengths)
    runs = [_runs(pos[t], doc[t]) for t in tokens]
    worst = 0
    for qr in runs:
        for kr in runs:
            n_shared = len(_full_spans(kr, shared_doc))
            for (_, ln, p0, d) in qr:
                n = int(np.count_nonzero((kr[:, 3] == d) & (kr[:, 2] <= p0 + ln - 1)))
                worst = max(worst, n + (n_shared if shared_doc >= 0 and int(d) != shared_doc else 0))
            if shared_doc >= 0:
                other = [(st, ln, p0, 1) for (st, ln, p0, d) in qr if int(d) != shared_doc]
                n_rows = len(_full_spans(other, 1))
                for (_, ln, p0, d) in kr:
                    if int(d) == shared_doc:
                        n = int(np.count_nonzero((qr[:, 3] == d) & (qr[:, 2] + qr[:, 1] - 1 >= p0)))
                        worst = max(worst, n + n_rows)
    return worst


def step_span_count(q_pos, q_doc, kv_pos, kv_doc, shared_doc: int = -1) -> int:
    """The most key spans one query run of this step meets: the block planner's limit is
    MAX_SPANS (the shared document's adjacent runs counted as one FULL span)."""
    qr, kr = _runs(np.asarray(q_pos), np.asarray(q_doc)), _runs(np.asarray(kv_pos), np.asarray(kv_doc))
    n_shared = len(_full_spans(kr, shared_doc))
    worst = 0
    for (_, ln, p0, d) in qr:
        n = int(np.count_nonzero((kr[:, 3] == d) & (kr[:, 2] <= p0 + ln - 1)))
        worst = max(worst, n + (n_shared if shared_doc >= 0 and int(d) != shared_doc else 0))
    return worst


def fused_span_count(q_pos, q_doc, kv_sides, shared_doc: int = -1) -> int:
    """The most key spans one query run meets over all the given steps together (the sum of
    its per-step counts, ``step_span_count``'s rule): a tile of a fused ring holds at most
    MAX_SPANS, so a ring fuses when this is within it."""
    qr = _runs(np.asarray(q_pos), np.asarray(q_doc))
    total = np.zeros(len(qr), dtype=np.int64)
    for kv_pos, kv_doc in kv_sides:
        kr = _runs(np.asarray(kv_pos), np.asarray(kv_doc))
        n_shared = len(_full_spans(kr, shared_doc))
        for i, (_, ln, p0, d) in enumerate(qr):
            total[i] += int(np.count_nonzero((kr[:, 3] == d) & (kr[:, 2] <= p0 + ln - 1)))
            total[i] += n_shared if shared_doc >= 0 and int(d) != shared_doc else 0
    return int(total.max()) if len(total) else 0


def _segments(doc, what):
    """(doc, start, length) of each maximal range of equal document id; a document must
    occupy one range (its tokens contiguous, as every sharding rule here leaves them)."""
    doc = np.asarray(doc)
    if len(doc) == 0:
        return []
    starts = np.r_[0, np.flatnonzero(np.diff(doc) != 0) + 1]
    ends = np.r_[starts[1:], len(doc)]
    seg = [(int(doc[a]), int(a), int(b - a)) for a, b in zip(starts, ends)]
    if len({d for d, _, _ in seg}) != len(seg):
        raise ValueError(f"{what}: a document's tokens are not contiguous")
    return seg


def step_slices(q_pos, q_doc, kv_pos, kv_doc, shared_doc: int = -1):
    """The block mask of one ring step as a slice list over local indices: key j visible to
    query i iff q_doc[i] == kv_doc[j] and kv_pos[j] <= q_pos[i], or kv_doc[j] == shared_doc !=
    q_doc[i].  Within each side a document's tokens are contiguous with ascending positions,
    so a row sees a prefix of its document's keys, c_i of them; rows where c grows by one per
    row are one CAUSAL rectangle (bottom-right aligned), rows of equal c one FULL rectangle,
    and each also gets a FULL rectangle over the shared document's keys.  Rows that see no
    key are left out (the plan gives them lse = -inf).  This is how a step whose query runs
    meet more than MAX_SPANS key runs (striped sharding: stripes of w tokens make a run per
    stripe) runs on the slice-list planner.  Returns (q_start, q_len, k_start, k_len, kind)."""
    from . import SLICE_CAUSAL, SLICE_FULL
    q_pos, kv_pos = np.asarray(q_pos, np.int64), np.asarray(kv_pos, np.int64)
    qs, ks = _segments(q_doc, "query shard"), _segments(kv_doc, "key/value shard")
    for side, pos in ((qs, q_pos), (ks, kv_pos)):
        for _, a, n in side:
            if n > 1 and np.any(np.diff(pos[a:a + n]) <= 0):
                raise ValueError("positions must ascend within a document")
    kv_of = {d: (a, n) for d, a, n in ks}
    shared = kv_of.get(shared_doc) if shared_doc >= 0 else None
    out = []
    for d, a, n in qs:
        own = kv_of.get(d)
        c = np.searchsorted(kv_pos[own[0]:own[0] + own[1]], q_pos[a:a + n], side="right") if own else np.zeros(n, int)
        sh = shared if shared is not None and d != shared_doc else None
        i = 0
        while i < n:
            j = i + 1
            step = int(c[j] - c[j - 1]) if j < n else None
            if step in (0, 1):
                while j < n and c[j] - c[j - 1] == step:
                    j += 1
            causal = step == 1 and j - i > 1
            k_len = int(c[j - 1]) if causal else int(c[i])
            rows = []
            if own is not None and k_len >= 1:
                rows.append((a + i, j - i, own[0], k_len, SLICE_CAUSAL if causal else SLICE_FULL))
            if sh is not None:
                rows.append((a + i, j - i, sh[0], sh[1], SLICE_FULL))
            out.extend(sorted(rows, key=lambda x: x[2]))
            i = j
    return out


def predicted_blocks(q_pos, q_doc, kv_pos, kv_doc, tile_rows: int) -> int:
    return predicted_work(q_pos, q_doc, kv_pos, kv_doc, tile_rows)[0]


def rank_work(lengths, tokens, tile_rows: int):
    """Per rank: (key blocks, work items, ring steps with any work), one kv head, over all
    its ring steps."""
    pos, doc = token_meta(lengths)
    cp = len(tokens)
    out = []
    for r in range(cp):
        b = i = s = 0
        for t in range(cp):
            src = tokens[ring_source(r, t, cp)]
            bt, it = predicted_work(pos[tokens[r]], doc[tokens[r]], pos[src], doc[src], tile_rows)
            b, i, s = b + bt, i + it, s + (it > 0)
        out.append((b, i, s))
    return out


# Rank time model: us = a * blocks * kv_heads / CUs + b * items * kv_heads / CUs + c * steps + d.
# Fitted (least squares, fit_cost.py) to the 32 rank shares of the 131072-token pack at cp = 8
# under zigzag, per-document and dispatch over 32 and 64 chunks, measured on one MI355X (256
# CUs, 32 q / 8 kv heads, d = 128, the steps' attention launches on 4 streams): within 8% of
# every one.  a matches the kernel's per-block time (1.85 us per 64-key block per workgroup).
TIME_MODEL_US = dict(per_block=1.808, per_item=15.526, per_step=32.888, fixed=132.966)


def predicted_rank_us(work, kv_heads: int, n_cu: int = 256, model=TIME_MODEL_US):
    return [model["per_block"] * b * kv_heads / n_cu + model["per_item"] * i * kv_heads / n_cu +
            model["per_step"] * s + model["fixed"] for (b, i, s) in work]


def parse_rule(name: str):
    """"dispatch/64" -> ("dispatch", 64); other names -> (name, 0)."""
    rule, _, n = name.partition("/")
    return rule, int(n) if n else 0


def choose_sharding(lengths, cp: int, tile_rows: int, kv_heads: int = 8, n_cu: int = 256,
                    rules=("zigzag", "per_document")):
    """The rule whose busiest rank has the smallest predicted time, with, per rule, the
    per-rank predicted microseconds and work: {rule: {"us": [...], "work": [(blocks, items,
    steps), ...]}}.  A rule is "zigzag", "per_document", or "dispatch/<chunks>"; rules that
    do not apply (zigzag and dispatch need the pack to divide evenly) or whose runs the
    planner would refuse (more than MAX_SPANS key runs per query run) are left out."""
    cost = {}
    for name in rules:
        rule, n = parse_rule(name)
        try:
            tokens = shard_tokens(rule, lengths, cp, n_chunks=n)
        except ValueError:
            continue
        if max_spans(lengths, tokens) > MAX_SPANS:
            continue
        work = rank_work(lengths, tokens, tile_rows)
        cost[name] = {"us": predicted_rank_us(work, kv_heads, n_cu), "work": work}
    best = min(cost, key=lambda r: max(cost[r]["us"]))
    return best, cost


# --------------------------------------------------------------------------
# device-resident shards and one rank's ring
# --------------------------------------------------------------------------
def build_shards(lengths, tokens, get_rows, device="cuda"):
    """Per rank: its tokens' q [n,H,d], stacked k/v [2,n,H_kv,d] (bf16) and positions and
    document ids (int32), on the device.  get_rows(idx) -> (q, k, v) of the given global
    token indices, as bf16 bit arrays (uint16) or bf16 tensors."""
    pos, doc = token_meta(lengths)

    def bf16(x):
        if isinstance(x, torch.Tensor):
            return x.to(device=device, dtype=torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)

    shards = []
    for idx in tokens:
        q, k, v = get_rows(idx)
        shards.append(dict(tokens=idx, q=bf16(q).contiguous(), kv=torch.stack([bf16(k), bf16(v)]).contiguous(),
                           pos=torch.from_numpy(pos[idx]).to(device), doc=torch.from_numpy(doc[idx]).to(device)))
    return shards


def live_steps(q_pos, q_doc, kv_sides, shared_doc: int = -1):
    """Indices of the (kv_pos, kv_doc) sides with at least one key some query row sees:
    the planner's work items for them are not all empty."""
    return [t for t, (kp, kd) in enumerate(kv_sides) if predicted_work(q_pos, q_doc, kp, kd, 64, shared_doc)[1] > 0]


class ShardedRank:
    """One rank's cp ring steps over device-resident shards (see ``build_shards``).

    run() calls block_attn_fwd per step (planning each); run_planned() plans every step
    in one launch first; run_overlapped() also lets the steps' attention launches overlap;
    capture()/replay() record either in a HIP graph.  Results are out (fp32 [n_q,H,d]) and
    lse ([H,n_q]) of the rank's tokens, in their order.

    A step whose chunk holds no key any of the rank's rows sees (judged on the host from the
    positions and document ids, which the sharding fixes before any data moves: the same
    tile count as the planner's, ``predicted_work``) runs nothing: no plan, no attention
    launch, no merge.  Merging it would change no bit (a partial whose lse is -inf leaves
    the running result as it is), so ``live_steps`` lists the steps that run.
    """

    def __init__(self, shards, rank, device="cuda", shared_doc=-1):
        from . import new_workspace
        cp = len(shards)
        self.cp, self.rank = cp, rank
        self.shared_doc = shared_doc  # a document every other document's rows see in full, or -1
        me = shards[rank]
        self.tokens = me["tokens"]
        self.q, self.q_pos, self.q_doc = me["q"], me["pos"], me["doc"]
        self.steps = []
        for t in range(cp):
            src = shards[ring_source(rank, t, cp)]
            self.steps.append(dict(source=ring_source(rank, t, cp), kv=src["kv"], kv_pos=src["pos"],
                                   kv_doc=src["doc"]))
        n_q, H, d = self.q.shape
        Hkv = self.steps[0]["kv"].shape[2]
        self.out = torch.empty((n_q, H, d), dtype=torch.float32, device=device)
        self.lse = torch.empty((H, n_q), dtype=torch.float32, device=device)
        self.step_out = torch.empty_like(self.out)
        self.step_lse = torch.empty_like(self.lse)
        # workspace sized for the longest side and the most runs of any step
        n_max = max([n_q] + [s["kv"].shape[1] for s in self.steps])
        runs = max([len(_runs(self.q_pos.cpu().numpy(), self.q_doc.cpu().numpy()))] +
                   [len(_runs(s["kv_pos"].cpu().numpy(), s["kv_doc"].cpu().numpy())) for s in self.steps])
        self._ws_shape = (n_max, max(1, runs), H, Hkv, device)
        self.workspace = new_workspace(*self._ws_shape)
        qp, qd = self.q_pos.cpu().numpy(), self.q_doc.cpu().numpy()
        self.live_steps = live_steps(qp, qd, [(s["kv_pos"].cpu().numpy(), s["kv_doc"].cpu().numpy())
                                              for s in self.steps], shared_doc)
        # a live step whose query runs meet more key runs than the block planner takes
        # (striped shards) runs as a slice list: same mask, planned by the slice-list planner
        for t in self.live_steps:
            st = self.steps[t]
            kp, kd = st["kv_pos"].cpu().numpy(), st["kv_doc"].cpu().numpy()
            if step_span_count(qp, qd, kp, kd, shared_doc) > MAX_SPANS:
                sl = step_slices(qp, qd, kp, kd, shared_doc)
                st["slices"] = torch.tensor(sl, dtype=torch.int32, device=device).reshape(-1, 5)
        self.step_workspaces = None
        self.graph = None
        self.overlap_buffers = None
        self._set_fusable(qp, qd)

    def _set_fusable(self, q_pos, q_doc):
        """The live steps can run as a fused ring (run_fused) when they are all block steps and
        no query run meets more than MAX_SPANS key runs over all of them together."""
        live_sides = [(self.steps[t]["kv_pos"].cpu().numpy(), self.steps[t]["kv_doc"].cpu().numpy())
                      for t in self.live_steps]
        # the fused planner takes at most FUSED_TILE_CAP query tiles; bounded here with the
        # shortest tile either the forward or the backward's dQ side cuts (32 rows)
        q_tiles = int(np.sum(-(-_runs(np.asarray(q_pos), np.asarray(q_doc))[:, 1] // 32)))
        self.fusable = bool(self.live_steps) and not any("slices" in self.steps[t] for t in self.live_steps) and \
            fused_span_count(q_pos, q_doc, live_sides, self.shared_doc) <= MAX_SPANS and q_tiles <= FUSED_TILE_CAP

    def _no_live_step(self):
        """The result when no step has a visible pair: every row sees nothing."""
        self.out.zero_()
        self.lse.fill_(-float("inf"))
        return self.out, self.lse

    def _new_step_workspace(self, t):
        from . import new_workspace
        st = self.steps[t]
        if "slices" in st:
            n_q, H, _ = self.q.shape
            return new_workspace(n_q, 2 * st["slices"].shape[0] + 1, H, st["kv"].shape[2], self.q.device)
        return new_workspace(*self._ws_shape)

    def run(self, stream=None, per_step=None):
        """Every live step, each a block_attn_fwd (or, for a slice-list step, its plan and
        run), and a merge for each after the first."""
        from . import attn_run, block_attn_fwd, lse_merge, plan_slices
        if not self.live_steps:
            return self._no_live_step()
        n_q, H, d = self.q.shape
        for i, t in enumerate(self.live_steps):
            st = self.steps[t]
            first = i == 0
            out = self.out if first else self.step_out
            lse = self.lse if first else self.step_lse
            if "slices" in st:
                if self.step_workspaces is None:
                    self.step_workspaces = [self._new_step_workspace(u) if u in self.live_steps else None
                                            for u in range(len(self.steps))]
                ws = plan_slices(st["slices"], n_q, st["kv"].shape[1], H, st["kv"].shape[2], d,
                                 workspace=self.step_workspaces[t], stream=stream)
                attn_run(self.q, st["kv"][0], st["kv"][1], out, lse, ws, stream=stream)
            else:
                block_attn_fwd(self.q, st["kv"], self.q_pos, st["kv_pos"], self.q_doc, st["kv_doc"], out=out,
                               lse=lse, workspace=self.workspace, stream=stream, shared_doc=self.shared_doc)
            if per_step is not None:
                per_step(t, out, lse)
            if not first:
                lse_merge(self.out, self.lse, self.step_out, self.step_lse, stream=stream)
        return self.out, self.lse

    def plan_all(self, stream=None):
        """Plans every live ring step in one launch, one workspace per step (None for the
        others): a step's key/value positions and document ids follow from the sharding,
        before its data arrive."""
        from . import plan_block_steps, plan_slices
        if self.step_workspaces is None:
            self.step_workspaces = [self._new_step_workspace(t) if t in self.live_steps else None
                                    for t in range(len(self.steps))]
        if not self.live_steps:
            return
        n_q, H, d = self.q.shape
        Hkv = self.steps[0]["kv"].shape[2]
        by_runs = [t for t in self.live_steps if "slices" not in self.steps[t]]
        if by_runs:
            live = [self.steps[t] for t in by_runs]
            plan_block_steps(self.q_pos, self.q_doc, [st["kv_pos"] for st in live], [st["kv_doc"] for st in live], H,
                             Hkv, d, [self.step_workspaces[t] for t in by_runs], stream=stream,
                             shared_doc=self.shared_doc)
        for t in self.live_steps:
            st = self.steps[t]
            if "slices" in st:
                plan_slices(st["slices"], n_q, st["kv"].shape[1], H, Hkv, d, workspace=self.step_workspaces[t],
                            stream=stream)

    def run_planned(self, stream=None, per_step=None):
        """run() with the plans of all live steps made up front by plan_all(): one planning
        launch, then per step the attention launch and (after the first) the merge."""
        from . import attn_run, lse_merge
        if not self.live_steps:
            return self._no_live_step()
        self.plan_all(stream)
        for i, t in enumerate(self.live_steps):
            st = self.steps[t]
            first = i == 0
            out = self.out if first else self.step_out
            lse = self.lse if first else self.step_lse
            attn_run(self.q, st["kv"][0], st["kv"][1], out, lse, self.step_workspaces[t], stream=stream)
            if per_step is not None:
                per_step(t, out, lse)
            if not first:
                lse_merge(self.out, self.lse, self.step_out, self.step_lse, stream=stream)
        return self.out, self.lse

    def run_overlapped(self, streams, stream=None):
        """run_planned() with step t's attention launch on streams[t % len(streams)], so
        that the workgroups of one step take the compute units that the previous step
        leaves idle while its last items finish (a persistent launch ends with a tail
        whose length is set by its largest items, not by its total work).  Every step
        writes its own partial buffers; the merges then run in step order on the
        calling stream, each once its step is done: the same kernels on the same data
        as run_planned(), so the same bits."""
        from . import attn_run, lse_merge
        main = torch.cuda.current_stream() if stream is None else stream
        if not self.live_steps:
            with torch.cuda.stream(main):
                return self._no_live_step()
        if self.overlap_buffers is None:
            self.overlap_buffers = [(self.out, self.lse)] + [
                (torch.empty_like(self.out), torch.empty_like(self.lse)) for _ in self.live_steps[1:]]
        self.plan_all(main)
        planned = torch.cuda.Event()
        planned.record(main)
        done = []
        for i, t in enumerate(self.live_steps):
            st = self.steps[t]
            s = streams[i % len(streams)]
            s.wait_event(planned)
            out, lse = self.overlap_buffers[i]
            attn_run(self.q, st["kv"][0], st["kv"][1], out, lse, self.step_workspaces[t], stream=s)
            ev = torch.cuda.Event()
            ev.record(s)
            done.append(ev)
        main.wait_event(done[0])
        for i in range(1, len(self.live_steps)):
            main.wait_event(done[i])
            lse_merge(self.out, self.lse, *self.overlap_buffers[i], stream=main)
        return self.out, self.lse

    def backward(self, dout, stream=None, ring=False, fused=False):
        """The rank's ring backward after a forward (run, run_planned, run_overlapped or a
        replay) left out and lse: D = <dout, out> once, then per live step the query shard's
        dq contribution (added into one fp32 buffer, so the steps run in order) and the source
        chunk's partial dk, dv, each in its own buffer -- what the rank would send back to
        the chunk's owner ("03 · 长文负载均衡", section 4.4: partial key/value gradients are
        reduced at the owning rank).  dout: bf16 [n_q, H, d] in the rank's token order.
        Returns dq (fp32 [n_q, H, d]) and the list of per-step dkv (fp32 [2, n_kv, H_kv, d]),
        None for a step no row sees: it sends nothing back.  ring=True runs the live steps'
        dK/dV items in one launch from one longest-first queue (lb_block_attn_bwd_ring); dq
        is added step after step either way."""
        from . import LBError, attn_bwd_rowdot, block_attn_bwd
        if any("slices" in self.steps[t] for t in self.live_steps):
            raise LBError("the backward of a ring step planned as a slice list (a step whose query runs meet more "
                          f"than {MAX_SPANS} key runs, e.g. striped shards) is not built")
        if getattr(self, "bwd_buffers", None) is None:
            n_q, H, d = self.q.shape
            ws_bytes = 2 * self.workspace.numel() + 512
            self.bwd_buffers = dict(
                dvec=torch.empty((H, n_q), dtype=torch.float32, device=self.q.device),
                dq=torch.empty((n_q, H, d), dtype=torch.float32, device=self.q.device),
                dkv=[torch.empty((2,) + tuple(st["kv"].shape[1:]), dtype=torch.float32, device=self.q.device)
                     for st in self.steps],
                ws=[torch.empty(ws_bytes, dtype=torch.uint8, device=self.q.device) for _ in self.steps])
        b = self.bwd_buffers
        attn_bwd_rowdot(self.out, dout, dvec=b["dvec"], stream=stream)
        b["dq"].zero_()
        if ring and self.live_steps:
            from . import block_attn_bwd_ring, new_ring_workspace
            if getattr(self, "bwd_ring_workspace", None) is None:
                n_max, runs, H, Hkv, device = self._ws_shape
                self.bwd_ring_workspace = new_ring_workspace(len(self.live_steps), n_max, runs, H, Hkv, device=device)
            live = self.live_steps
            q_ring = None
            if fused:  # the dQ side as a fused ring: one launch, each query tile against every step
                if not self.fusable:
                    raise ValueError("this share's live steps do not fuse")
                if getattr(self, "bwd_q_ring_workspace", None) is None:
                    n_max, runs, H, Hkv, device = self._ws_shape
                    self.bwd_q_ring_workspace = new_ring_workspace(len(self.live_steps), n_max, runs, H, Hkv,
                                                                   device=device)
                q_ring = self.bwd_q_ring_workspace
            block_attn_bwd_ring(self.q, [self.steps[t]["kv"] for t in live], dout, self.lse, b["dvec"], self.q_pos,
                                self.q_doc, [self.steps[t]["kv_pos"] for t in live],
                                [self.steps[t]["kv_doc"] for t in live], b["dq"], [b["dkv"][t] for t in live],
                                [b["ws"][t] for t in live], self.bwd_ring_workspace, stream=stream,
                                shared_doc=self.shared_doc, q_ring_workspace=q_ring)
            return b["dq"], [b["dkv"][t] if t in live else None for t in range(len(self.steps))]
        for t in self.live_steps:
            st = self.steps[t]
            block_attn_bwd(self.q, st["kv"], dout, self.lse, b["dvec"], self.q_pos, st["kv_pos"], self.q_doc,
                           st["kv_doc"], b["dq"], dkv=b["dkv"][t], workspace=b["ws"][t], stream=stream,
                           shared_doc=self.shared_doc)
        return b["dq"], [b["dkv"][t] if t in self.live_steps else None for t in range(len(self.steps))]

    def plan_ring(self, stream=None):
        """plan_all(), then the live steps' plans merged into one longest-first queue in the
        ring workspace (allocated on first use, with the steps' partial buffers)."""
        from . import new_ring_workspace, plan_ring
        if self.overlap_buffers is None:
            self.overlap_buffers = [(self.out, self.lse)] + [
                (torch.empty_like(self.out), torch.empty_like(self.lse)) for _ in self.live_steps[1:]]
        live = [self.steps[t] for t in self.live_steps]
        if getattr(self, "ring_workspace", None) is None:
            n_max, runs, H, Hkv, device = self._ws_shape
            frags = max([runs] + [2 * st["slices"].shape[0] + 1 for st in live if "slices" in st])
            self.ring_workspace = new_ring_workspace(len(live), n_max, frags, H, Hkv, device=device)
        n_q, H, d = self.q.shape
        self.plan_all(stream)
        plan_ring([self.step_workspaces[t] for t in self.live_steps], [st["kv"].shape[1] for st in live], n_q, H,
                  live[0]["kv"].shape[2], d, self.ring_workspace, stream=stream)

    def ring_attention(self, stream=None):
        """The one attention launch over the ring workspace: live step i's partial into
        overlap_buffers[i] (the first is out, lse themselves)."""
        from . import ring_attn_run
        live = [self.steps[t] for t in self.live_steps]
        ring_attn_run(self.q, [st["kv"][0] for st in live], [st["kv"][1] for st in live],
                      [b[0] for b in self.overlap_buffers], [b[1] for b in self.overlap_buffers],
                      self.ring_workspace, stream=stream)

    def merge_partials(self, stream=None):
        """Merges the live steps' partials 1, 2, ... into out, lse in step order, in one pass
        (the same bits as a merge per step)."""
        from . import lse_merge_parts
        if len(self.live_steps) > 1:
            lse_merge_parts([b[0] for b in self.overlap_buffers], [b[1] for b in self.overlap_buffers],
                            stream=stream)

    def run_ring(self, stream=None):
        """run_planned() with every live step's items in one attention launch: the steps'
        plans (one planning launch) are merged into one longest-first queue, one persistent
        launch runs it, each step's partial into its own buffers, and the merges follow in
        step order.  A light step then adds its items to the common queue instead of a
        launch whose end waits for its largest items.  Each item computes what it computes
        in its own step's launch, so the result has the same bits as run_planned()."""
        if not self.live_steps:
            return self._no_live_step()
        self.plan_ring(stream)
        self.ring_attention(stream)
        self.merge_partials(stream)
        return self.out, self.lse

    def plan_ring_fused(self, stream=None):
        """plan_all(), then the live steps' plans fused per query tile in the ring workspace."""
        from . import new_ring_workspace, plan_ring
        if not self.fusable:
            raise ValueError("this share's live steps do not fuse (a slice-list step, or a query run meeting "
                             f"more than {MAX_SPANS} key runs over all of them)")
        live = [self.steps[t] for t in self.live_steps]
        if getattr(self, "ring_workspace", None) is None:
            n_max, runs, H, Hkv, device = self._ws_shape
            self.ring_workspace = new_ring_workspace(len(live), n_max, runs, H, Hkv, device=device)
        n_q, H, d = self.q.shape
        self.plan_all(stream)
        plan_ring([self.step_workspaces[t] for t in self.live_steps], [st["kv"].shape[1] for st in live], n_q, H,
                  live[0]["kv"].shape[2], d, self.ring_workspace, stream=stream, fused=True)

    def run_fused(self, stream=None):
        """The share as a fused ring: one item per query tile and kv head runs the tile's rows
        against the keys of every live step in one online softmax and writes out, lse
        directly.  No partials, no merges; equal to run_ring() to the rounding of the bf16 softmax
        weights (each path rounds them against its own running maximum)."""
        from . import ring_attn_run_fused
        if not self.live_steps:
            return self._no_live_step()
        self.plan_ring_fused(stream)
        live = [self.steps[t] for t in self.live_steps]
        ring_attn_run_fused(self.q, [st["kv"][0] for st in live], [st["kv"][1] for st in live], self.out, self.lse,
                            self.ring_workspace, stream=stream)
        return self.out, self.lse

    def capture(self, stream=None, streams=None, ring=False, fused=False):
        """Captures run_planned() -- one planning launch, an attention launch per live step and
        a merge for each after the first -- or, given side streams, run_overlapped(), or with
        ring=True run_ring(), into a HIP graph, so that
        replay() launches the whole share at once.  Every kernel of the share is safe to
        replay: the planner resets the queue heads and the attention kernel rewinds them,
        and nothing in it clears memory with a memset node."""
        if fused:
            body = lambda st=None: self.run_fused(stream=st)
        elif ring:
            body = lambda st=None: self.run_ring(stream=st)
        else:
            body = (lambda st=None: self.run_planned(stream=st)) if streams is None else \
                (lambda st=None: self.run_overlapped(streams, stream=st))
        body(stream)  # allocates the step workspaces and buffers, caches the CU count
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body()
        torch.cuda.synchronize()
        self.graph = g
        return g

    def replay(self):
        """One launch of the captured share; returns (out, lse), written in place."""
        self.graph.replay()
        return self.out, self.lse
