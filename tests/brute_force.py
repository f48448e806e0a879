"""Pure-Python attention for tiny inputs: nested loops and math.exp.

Written independently of ``oracle/`` (no numpy linear algebra, no shared
helpers) so that it pins the oracle: a transposed operand, a dropped scale, a
wrong mask direction or a wrong head mapping in the oracle would make the two
disagree.  The definition is the unfused chain of the Step 3.7 page §2.3:
s_ij = scale * sum_c q_ic k_jc (+ mask_ij), p_ij = exp(s_ij) / sum_j exp(s_ij),
o_ic = sum_j p_ij v_jc.
"""
import math


def attention(q, k, v, scale, causal=False, mask=None, kv_len=None):
    """q: list of Nq rows, k/v: lists of Nk rows (lists of floats).

    Returns (o rows, lse list).  mask: Nq x Nk list or None.
    """
    nq, nk, d = len(q), len(k), len(q[0])
    out, lses = [], []
    for i in range(nq):
        logits = []
        for j in range(nk):
            visible = True
            if kv_len is not None and j >= kv_len:
                visible = False
            if causal and j > i:
                visible = False
            if not visible:
                logits.append(None)
                continue
            dot = 0.0
            for c in range(d):
                dot += q[i][c] * k[j][c]
            x = dot * scale
            if mask is not None:
                x += mask[i][j]
            logits.append(x)
        vis = [x for x in logits if x is not None and x != -math.inf]
        if not vis:
            out.append([0.0] * d)
            lses.append(-math.inf)
            continue
        big = max(vis)
        w = [0.0 if (x is None or x == -math.inf) else math.exp(x - big) for x in logits]
        tot = sum(w)
        row = []
        for c in range(d):
            acc = 0.0
            for j in range(nk):
                acc += w[j] * v[j][c]
            row.append(acc / tot)
        out.append(row)
        lses.append(big + math.log(tot))
    return out, lses
