"""Oracle: packed zigzag split and branch index (test infrastructure only).

Definitions followed (pages of arXiv:2609.07108):

* rainbus analysis, background section on context parallelism: zigzag
  sharding gives every rank both a head chunk and a tail chunk of the
  sequence so that causal work is balanced; "packed" means variable-length
  sequences are concatenated without padding to a common length.
* rainbus analysis, method steps, step two: the main sequence is packed into
  zigzag chunks and each of the C ranks holds N/C tokens.
* ai.info summary, Key Contributions 1 and Methodology: the branch-local part
  lives on the rank that owns the branch's anchor.

Readings where the pages are silent:

* every sequence is padded at its tail to a multiple of 2C and cut into 2C
  equal chunks; rank r holds chunks r and 2C-1-r, in that order, sequences in
  batch order (the tiny EAGLE-3 workload pins rank 0 of C=2 to chunks {0,3});
* pad positions carry no keys and their query rows see nothing;
* anchors are global indices into the packed stream of real tokens; for
  EAGLE-3 TTT every real position is an anchor with ``depth`` branch rows;
  local anchors are ordered by their local main row;
* branch rows (and branch keys) of the local anchors are stored back to back
  in local-anchor order, ``branch_off`` giving each anchor's first row.

Parity: pinned (tests/test_oracle_pack.py: golden layout of the tiny
workload, bijection over ranks, closed-form pair counts).
"""

import numpy as np

KIND_NONE = 0
KIND_TTT = 1
KIND_BLOCK_BIDIR = 2
KIND_BLOCK_CAUSAL = 3


def zigzag_layout(seqlens, C, r):
    """Zigzag split of packed sequences for rank ``r`` of ``C``.

    Returns a dict of int64 arrays:
      L, P, c            per sequence: real length, padded length, chunk size
      cu_real, cu_pad    prefix sums of L and P (length S+1)
      cu_local           prefix sums of local rows (2c per sequence)
      pos, seq           per local row: position inside its sequence, sequence
      perm               per local row: global padded position cu_pad[seq]+pos
      is_pad             per local row: 1 if pos >= L[seq]
    and the scalars C, r, n_local.
    """
    L = np.asarray(seqlens, dtype=np.int64)
    if L.ndim != 1 or L.size == 0 or np.any(L < 1):
        raise ValueError("seqlens must be a non-empty list of positive lengths")
    if not (1 <= C) or not (0 <= r < C):
        raise ValueError("need C >= 1 and 0 <= r < C")
    two_c = 2 * C
    P = ((L + two_c - 1) // two_c) * two_c
    c = P // two_c
    cu_real = np.concatenate([[0], np.cumsum(L)])
    cu_pad = np.concatenate([[0], np.cumsum(P)])
    cu_local = np.concatenate([[0], np.cumsum(2 * c)])
    pos_parts, seq_parts = [], []
    for s in range(L.size):
        head = np.arange(r * c[s], (r + 1) * c[s])
        tail = np.arange((two_c - 1 - r) * c[s], (two_c - r) * c[s])
        pos_parts.append(np.concatenate([head, tail]))
        seq_parts.append(np.full(2 * c[s], s))
    pos = np.concatenate(pos_parts).astype(np.int64)
    seq = np.concatenate(seq_parts).astype(np.int64)
    return dict(
        C=C, r=r, n_local=int(cu_local[-1]),
        L=L, P=P, c=c,
        cu_real=cu_real, cu_pad=cu_pad, cu_local=cu_local,
        pos=pos, seq=seq,
        perm=cu_pad[seq] + pos,
        is_pad=(pos >= L[seq]).astype(np.int64),
    )


def shard_positions(layout, shard):
    """Per-row (sequence, position) of K/V shard ``shard``: rank ``shard``'s own
    local row order (the K/V block that rank ``shard`` holds and sends around
    the ring)."""
    other = zigzag_layout(layout["L"], layout["C"], shard)
    return other["seq"], other["pos"]


def branch_index(layout, kind, depth_or_block=0, anchors=None, branch_lens=None):
    """Anchor -> branch map for the layout's rank.

    ``kind``: KIND_NONE, KIND_TTT (every real position anchors ``depth_or_block``
    chained rows), KIND_BLOCK_BIDIR or KIND_BLOCK_CAUSAL (``anchors`` are global
    real-token indices, strictly increasing; ``branch_lens`` per anchor, or the
    uniform ``depth_or_block``).

    Returns int64 arrays anchor_row, anchor_pos, anchor_seq, branch_off (A+1),
    and per branch row: b_anchor (local anchor id), b_j (index in its branch),
    b_len (its branch's length); plus the scalar kind.
    """
    L, cu_real = layout["L"], layout["cu_real"]
    C, c = layout["C"], layout["c"]
    if kind == KIND_NONE:
        glob = np.zeros(0, dtype=np.int64)
        lens = np.zeros(0, dtype=np.int64)
    elif kind == KIND_TTT:
        if depth_or_block < 1:
            raise ValueError("TTT depth must be >= 1")
        glob = np.arange(int(cu_real[-1]), dtype=np.int64)
        lens = np.full(glob.size, depth_or_block, dtype=np.int64)
    elif kind in (KIND_BLOCK_BIDIR, KIND_BLOCK_CAUSAL):
        glob = np.asarray(anchors, dtype=np.int64)
        if glob.size and (np.any(np.diff(glob) <= 0) or glob[0] < 0 or glob[-1] >= cu_real[-1]):
            raise ValueError("anchors must be strictly increasing real-token indices")
        if branch_lens is None:
            lens = np.full(glob.size, depth_or_block, dtype=np.int64)
        else:
            lens = np.asarray(branch_lens, dtype=np.int64)
        if lens.size != glob.size or np.any(lens < 1):
            raise ValueError("one positive branch length per anchor")
    else:
        raise ValueError("unknown branch kind")

    # which sequence and position each global anchor falls on
    a_seq = np.searchsorted(cu_real, glob, side="right") - 1
    a_pos = glob - cu_real[a_seq]
    # chunk of that position and the rank holding it
    chunk = a_pos // c[a_seq]
    owner = np.where(chunk < C, chunk, 2 * C - 1 - chunk)
    mine = owner == layout["r"]
    a_seq, a_pos, lens, chunk = a_seq[mine], a_pos[mine], lens[mine], chunk[mine]
    # local main row of each kept anchor
    in_head = chunk < C
    within = a_pos - chunk * c[a_seq]
    row = layout["cu_local"][a_seq] + np.where(in_head, within, c[a_seq] + within)
    order = np.argsort(row, kind="stable")
    row, a_pos, a_seq, lens = row[order], a_pos[order], a_seq[order], lens[order]
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    nb = int(off[-1])
    b_anchor = np.repeat(np.arange(row.size, dtype=np.int64), lens)
    b_j = np.arange(nb, dtype=np.int64) - off[b_anchor]
    return dict(
        kind=kind,
        anchor_row=row.astype(np.int64), anchor_pos=a_pos.astype(np.int64),
        anchor_seq=a_seq.astype(np.int64), branch_off=off,
        b_anchor=b_anchor, b_j=b_j, b_len=lens[b_anchor] if nb else np.zeros(0, np.int64),
        n_branch=nb,
    )


def pair_counts(layout, br):
    """Unmasked (query row, key) pairs per q-head, split into main rows,
    branch rows' main prefix, and branch-local keys, counted straight from the
    visibility rules (main row at p sees p+1 keys; branch row of an anchor at
    p_a sees p_a+1 main keys plus its own branch keys)."""
    real = layout["is_pad"] == 0
    main = int(np.sum(layout["pos"][real] + 1))
    if br["n_branch"] == 0:
        return dict(main=main, prefix=0, local=0, total=main)
    prefix = int(np.sum(br["anchor_pos"][br["b_anchor"]] + 1))
    if br["kind"] == KIND_BLOCK_BIDIR:
        local = int(np.sum(br["b_len"]))
    else:
        local = int(np.sum(br["b_j"] + 1))
    return dict(main=main, prefix=prefix, local=local, total=main + prefix + local)
