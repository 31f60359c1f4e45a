"""Nested-loop formulation of the all-to-allv dispatch, for small inputs only.

TEST INFRASTRUCTURE ONLY (see the package docstring).  This is a second way of writing
the definition that the C oracle implements with a counting sort and offset tables.  It
uses no counts, no prefix sums and no positions: it appends rows to lists in the order
the definition fixes, so a mistake in the C oracle's offsets or cursors cannot also be
here.  Pure Python: only for inputs of a few tokens.

Definition (abhik.ai "Collective Communication for 100k+ GPUs", section "Inference:
small messages, unknown sizes", Figure 13): each rank sorts its (token, slot)
assignments by expert into a send buffer and an all-to-allv delivers each row to the
rank holding its expert.  Readings: owner(e) = e // experts_per_rank; the sort is stable
in (expert, token, slot); rank d's receive buffer is the concatenation over source
ranks s = 0..R-1 of the rows s sends to d, in s's send order.
"""


def send_lists(ids, R, T, k, epr):
    """send[s] = list of (t, j) in send-buffer order, built expert by expert."""
    E = R * epr
    out = []
    for s in range(R):
        lst = []
        for e in range(E):
            for t in range(T):
                for j in range(k):
                    if int(ids[s][t][j]) == e:
                        lst.append((t, j))
        out.append(lst)
    return out


def recv_lists(ids, R, T, k, epr):
    """recv[d] = list of (s, t, j, e) in receive-buffer order, built by nested loops:
    for each destination d, each source s, each expert e of d, each token t, slot j."""
    out = []
    for d in range(R):
        lst = []
        for s in range(R):
            for e in range(d * epr, (d + 1) * epr):
                for t in range(T):
                    for j in range(k):
                        if int(ids[s][t][j]) == e:
                            lst.append((s, t, j, e))
        out.append(lst)
    return out


def recv_lists_expert_major(ids, R, T, k, epr):
    """recv[d] in the expert-major layout: for each destination d, each expert e of d,
    each source s, each token t, slot j."""
    out = []
    for d in range(R):
        lst = []
        for e in range(d * epr, (d + 1) * epr):
            for s in range(R):
                for t in range(T):
                    for j in range(k):
                        if int(ids[s][t][j]) == e:
                            lst.append((s, t, j, e))
        out.append(lst)
    return out
