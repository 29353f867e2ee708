"""CPU model of the address arithmetic of the decode and merge kernels.

Test infrastructure: a plain-Python restatement of the index math in
csrc/mfma_common.h (schedule_start), csrc/decode_mfma.hip (the tile cursor, the
staging addresses, the packed-row map and the partial slots of finish_segment),
csrc/merge.hip (the persistent merge's ownership and slot choice) and
csrc/decode_valu.hip (the split-K grid), evaluated on the host for the plans that
gqa_decode_plan returns. It checks, for every workgroup of a plan, what a GPU run
would only show as a fault or a silently wrong row:

* every (sequence, group, row block, tile) is consumed by exactly one workgroup;
* every cache row, block-table entry and page a tile touches lies inside its buffer
  (only the table entries below ceil(L / P) are read, as the header promises), the
  entries of the tile after a workgroup's last one included (they are loaded one
  pipeline step ahead);
* a plain-path staging load never straddles a page, and the entry loaded ahead for
  its 16-row group is its page;
* every partial row a workgroup writes lies inside the workspace the plan sizes, no
  (workgroup, slot) is written twice, and only a segment cut by a workgroup boundary
  writes one;
* the merge reads, for each cut segment, exactly the partials the decode kernel wrote
  for it, and nothing else;
* the packed rows of each (sequence, group) cover that group's (token, head) rows of
  `out` exactly once.

The model walks segments, not single tiles, so that the full-size shapes of the
benchmark (about a million tiles) check in well under a second.
"""
from __future__ import annotations

from dataclasses import dataclass, field

T_MFMA = 32          # keys per tile of the persistent schedule
WS_ALIGN = 256       # workspace sub-buffer alignment


def clamp_len(L: int, capacity: int) -> int:
    return 1 if L < 1 else (capacity if L > capacity else L)


def round_up(x: int, a: int) -> int:
    return (x + a - 1) // a * a


def tile_lo(w: int, W: int, nwg: int) -> int:
    return (w * W) // nwg


def tile_owner(f: int, W: int, nwg: int) -> int:
    """Largest w with tile_lo(w) <= f (the merge's closed form)."""
    return ((f + 1) * nwg - 1) // W


@dataclass
class Shape:
    B: int
    H: int
    G: int
    d_h: int
    q_len: int
    seq_lens: list
    capacity: int            # tokens per sequence (max_blocks * P when paged)
    page_size: int = 0       # 0: contiguous
    num_pages: int = 0
    max_blocks: int = 0


@dataclass
class Report:
    tiles: int = 0
    partial_writes: int = 0
    merged_segments: int = 0
    max_ws_row: int = -1
    max_table_index: int = -1
    notes: list = field(default_factory=list)


class ModelError(AssertionError):
    pass


def _check(cond: bool, msg: str):
    if not cond:
        raise ModelError(msg)


def row_block_rows(R: int, n_rb: int) -> int:
    """Rows per block of a group split into n_rb blocks (the planner's rule: one
    block of R rows, else equal blocks rounded up to whole 16-row tiles)."""
    return R if n_rb == 1 else ((R + n_rb - 1) // n_rb + 15) // 16 * 16


def schedule(shape: Shape, n_rb: int, nwg: int):
    """schedule_start for every workgroup: W, the per-sequence prefix sums the first
    wave publishes, and each workgroup's (lo, count, b, pre, L)."""
    GS = shape.G * n_rb
    lens = [clamp_len(int(L), shape.capacity) for L in shape.seq_lens]
    prefix = [0]
    for L in lens:
        prefix.append(prefix[-1] + GS * ((L + T_MFMA - 1) // T_MFMA))
    W = prefix[-1]
    _check(W < 2 ** 31, "tile count overflows int32")
    starts = []
    b = 0
    for w in range(nwg):
        lo = tile_lo(w, W, nwg)
        hi = tile_lo(w + 1, W, nwg)
        while b < shape.B and prefix[b + 1] <= lo:
            b += 1
        if hi - lo <= 0 or b >= shape.B:
            starts.append((lo, hi - lo, -1, 0, 1))
        else:
            starts.append((lo, hi - lo, b, prefix[b], lens[b]))
    return W, prefix, lens, starts


def check_persistent(shape: Shape, plan: dict) -> Report:
    """Walk every workgroup of a persistent (matrix-core) plan and check the decode
    kernel's and the merge kernel's index math against the plan's buffers."""
    rep = Report()
    _check(plan["schedule"] == 1, "not a persistent plan")
    nwg = plan["workgroups"]
    n_rb = plan["row_blocks"]
    R = plan["rows"]
    _check(R == shape.H // shape.G * shape.q_len, "packed rows per group")
    rbr = row_block_rows(R, n_rb)
    _check(n_rb * rbr >= R and (n_rb - 1) * rbr < R, "row blocks do not tile the group")
    _check(plan["max_splits"] == 2, "two partial slots per workgroup")
    D = shape.d_h
    # workspace: ws_o [nwg, 2, rbr, D] f32, ws_lse [nwg, 2, rbr] f32, ws_prefix [B + 1] i32
    need = (round_up(nwg * 2 * rbr * D * 4, WS_ALIGN) + round_up(nwg * 2 * rbr * 4, WS_ALIGN)
            + round_up((shape.B + 1) * 4, WS_ALIGN))
    _check(plan["workspace_bytes"] >= need, f"workspace {plan['workspace_bytes']} < {need}")
    ws_rows = nwg * 2 * rbr

    W, prefix, lens, starts = schedule(shape, n_rb, nwg)
    GS = shape.G * n_rb
    P = shape.page_size
    paged = P > 0
    pshift = P.bit_length() - 1 if paged else 0
    CPR = D // 8
    RPL = 256 // CPR          # tile rows one 16-byte staging load covers

    # (b, seg) -> list of (w, slot) partials written; consumed tile counts per segment
    written: dict = {}
    consumed: dict = {}
    complete_seen: dict = {}

    def seg_tiles(b):
        return (lens[b] + T_MFMA - 1) // T_MFMA

    def check_segment_addresses(b, g, t_first, t_last):
        L = lens[b]
        n = seg_tiles(b)
        _check(0 <= t_first <= t_last < n, "tile index outside its segment")
        # the last tile's rows are clamped to L - 1 (masked re-reads)
        j_max = min(t_last * T_MFMA + T_MFMA - 1, L - 1)
        if paged:
            # table entries read: min(t0 + 16 gi, L - 1) >> pshift
            idx = min(t_last * T_MFMA + 16 * (T_MFMA // 16 - 1), L - 1) >> pshift
            _check(idx < (L + P - 1) // P, "block-table entry at or past ceil(L / P)")
            _check(idx < shape.max_blocks, "block-table entry past the row")
            rep.max_table_index = max(rep.max_table_index, idx)
            # the plain path: tiles wholly before L, when a load's rows share a page
            fast = L // T_MFMA
            if P >= RPL and t_first < fast:
                for n_ld in range(T_MFMA * CPR // 256):
                    t0 = t_first * T_MFMA
                    j0 = t0 + n_ld * RPL
                    _check((j0 >> pshift) == ((j0 + RPL - 1) >> pshift), "staging load straddles a page")
                    _check(j0 + RPL - 1 < L, "plain-path load past the end")
                    # the plain path takes the page of load n_ld from the prefetched entry
                    # of its 16-row group
                    _check((j0 >> pshift) == ((t0 + 16 * ((n_ld * RPL) >> 4)) >> pshift),
                           "prefetched entry is not the load's page")
        else:
            row = (b * shape.G + g) * shape.capacity + j_max
            _check(j_max < shape.capacity and row < shape.B * shape.G * shape.capacity,
                   "contiguous cache row out of bounds")

    for w, (lo, count, b, pre, L) in enumerate(starts):
        if count <= 0 or b < 0:
            _check(count <= 0, "a workgroup with tiles but no sequence")
            continue
        # the cursor at tile lo
        n = seg_tiles(b)
        _check(lens[b] == L, "start length")
        seg = (lo - pre) // n
        t = (lo - pre) - seg * n
        _check(0 <= seg < GS, "start segment")
        left = count
        first = True
        seg_from_start = t == 0
        while left > 0:
            _check(b < shape.B, "cursor ran past the last sequence")
            n = seg_tiles(b)
            take = min(left, n - t)
            g, rb = divmod(seg, n_rb)
            check_segment_addresses(b, g, t, t + take - 1)
            consumed[(b, seg)] = consumed.get((b, seg), 0) + take
            rep.tiles += take
            left -= take
            seg_end = t + take == n
            complete = seg_from_start and seg_end
            if complete:
                complete_seen[(b, seg)] = complete_seen.get((b, seg), 0) + 1
            else:
                _check(first or left == 0, "a segment inside a workgroup left a partial")
                slot = 0 if first else 1
                written.setdefault((b, seg), []).append((w, slot))
                for r_local in (0, rbr - 1):
                    prow = (w * 2 + slot) * rbr + r_local
                    _check(0 <= prow < ws_rows, "partial row outside the workspace")
                    rep.max_ws_row = max(rep.max_ws_row, prow)
                rep.partial_writes += 1
            first = False
            if not seg_end:   # the workgroup's last tile ends inside this segment
                t += take
                break
            # advance: next segment of b, else next sequence
            t = 0
            seg_from_start = True
            seg += 1
            if seg == GS:
                seg = 0
                b += 1
        # paged: the table entries of the tile after the workgroup's last one are loaded
        # ahead (the cursor stops there); that tile belongs to another workgroup's share
        if paged and b < shape.B:
            L = lens[b]
            _check(t < seg_tiles(b), "look-ahead tile outside its segment")
            for gi in range(T_MFMA // 16):
                idx = min(t * T_MFMA + 16 * gi, L - 1) >> pshift
                _check(idx < (L + P - 1) // P and idx < shape.max_blocks, "look-ahead table entry out of range")
                rep.max_table_index = max(rep.max_table_index, idx)
    _check(rep.tiles == W, f"consumed {rep.tiles} of {W} tiles")
    slots = [ws for v in written.values() for ws in v]
    _check(len(slots) == len(set(slots)), "a (workgroup, slot) written twice")
    for b in range(shape.B):
        for seg in range(GS):
            _check(consumed.get((b, seg), 0) == seg_tiles(b), f"segment {(b, seg)} not covered once")
            _check(((b, seg) in complete_seen) != ((b, seg) in written),
                   f"segment {(b, seg)} both finished and partial, or neither")

    # the persistent merge: one (segment, row) at a time, from the published prefix
    for b in range(shape.B):
        pre_b = prefix[b]
        n_b = (prefix[b + 1] - pre_b) // GS
        for gs in range(GS):
            s0 = pre_b + gs * n_b
            wa = tile_owner(s0, W, nwg)
            wb = tile_owner(s0 + n_b - 1, W, nwg)
            _check(tile_lo(wa, W, nwg) <= s0 < tile_lo(wa + 1, W, nwg), "merge owner of the first tile")
            _check(tile_lo(wb, W, nwg) <= s0 + n_b - 1 < tile_lo(wb + 1, W, nwg), "merge owner of the last tile")
            if wa == wb:
                _check((b, gs) in complete_seen, "merge skips a segment nobody finished")
                continue
            slot_a = 1 if tile_lo(wa, W, nwg) < s0 else 0
            reads = []
            for wv in range(wa, wb + 1):
                if tile_lo(wv, W, nwg) < tile_lo(wv + 1, W, nwg):   # the workgroup owns tiles
                    reads.append((wv, slot_a if wv == wa else 0))
            _check(sorted(reads) == sorted(written.get((b, gs), [])),
                   f"merge of segment {(b, gs)} reads {reads}, decode wrote {written.get((b, gs))}")
            rep.merged_segments += 1

    # packed rows -> (token, head): every row of `out` exactly once
    hpg = shape.H // shape.G
    seen = set()
    for g in range(shape.G):
        for rb in range(n_rb):
            for r_local in range(rbr):
                r = rb * rbr + r_local
                if r < R:
                    t, k = divmod(r, hpg)
                    h = g * hpg + k
                    _check(0 <= t < shape.q_len and 0 <= h < shape.H, "packed row maps outside out")
                    _check((t, h) not in seen, "two packed rows map to one output row")
                    seen.add((t, h))
    _check(len(seen) == shape.q_len * shape.H, "some output rows have no packed row")
    return rep


def check_split_grid(shape: Shape, plan: dict) -> Report:
    """The split-K grid (vector-ALU policy): grid (splits, G * row blocks, B), split s
    of sequence b covers keys [s chunk, min((s + 1) chunk, L)), partial row
    orow * max_splits + s, and the merge reads ceil(L / chunk) splits."""
    rep = Report()
    _check(plan["schedule"] == 0, "not a split-K plan")
    chunk = plan["chunk_tokens"]
    S = plan["max_splits"]
    _check(plan["grid"] == [S, shape.G * plan["row_blocks"], shape.B], "grid shape")
    _check(chunk % plan["tile_tokens"] == 0 and chunk > 0, "chunk is whole tiles")
    _check(S * chunk >= shape.capacity and (S - 1) * chunk < shape.capacity, "splits cover the capacity")
    rows = shape.B * shape.q_len * shape.H
    if S > 1:
        need = round_up(rows * S * shape.d_h * 4, WS_ALIGN) + round_up(rows * S * 4, WS_ALIGN)
        _check(plan["workspace_bytes"] >= need, "split-K workspace too small")
    for b in range(shape.B):
        L = clamp_len(int(shape.seq_lens[b]), shape.capacity)
        ns = min((L + chunk - 1) // chunk, S)
        covered = 0
        for s in range(S):
            start = s * chunk
            if start >= L:
                _check(s >= ns, "the merge reads a split the kernel skipped")
                continue
            _check(s < ns, "a written split the merge does not read")
            covered += min(start + chunk, L) - start
        _check(covered == L, "splits do not cover the sequence once")
        orow_max = (b * shape.q_len + shape.q_len - 1) * shape.H + shape.H - 1
        _check((orow_max * S + ns - 1) < rows * S, "partial row outside the workspace")
        if shape.page_size:
            _check((L - 1) >> (shape.page_size.bit_length() - 1) < shape.max_blocks, "table entry past the row")
        rep.tiles += (L + plan["tile_tokens"] - 1) // plan["tile_tokens"]
    return rep
