"""Pure-Python attention for tiny inputs: nested loops and math.exp.

Written independently of ``oracle/`` (no numpy linear algebra, no shared
helpers) so that it pins the oracle: a transposed operand, a dropped scale, a
wrong mask direction or a wrong head mapping in the oracle would make the two
disagree.  The definition is the unfused chain of the Step 3.7 page §2.3:
s_ij = scale * sum_c q_ic k_jc (+ mask_ij), p_ij = exp(s_ij) / sum_j exp(s_ij),
o_ic = sum_j p_ij v_jc.
"""
import math


def attention(q, k, v, scale, causal=False, mask=None, kv_len=None, softcap=None,
              window=None, grid=None, last_positions=False, with_probs=False):
    """q: list of Nq rows, k/v: lists of Nk rows (lists of floats).

    Returns (o rows, lse list), and with ``with_probs`` also the Nq x Nk
    softmax weights p_ij.  mask: Nq x Nk list or None.

    Local options: the query of row i sits at position p = i, or with
    ``last_positions`` at the (L - Nq + i)-th of the L valid keys.  softcap:
    logit -> softcap * tanh(logit / softcap) before the mask.  window =
    (left, right): keys p - left .. p + right (a negative bound is open).
    grid = (cols, nbr_rows, nbr_cols): token t is the cell (t // cols,
    t % cols) of a row-major grid, and a key is visible when both its row
    and its column are nearer than nbr_rows / nbr_cols to the query's.
    """
    nq, nk, d = len(q), len(k), len(q[0])
    L = nk if kv_len is None else kv_len
    out, lses, probs = [], [], []
    for i in range(nq):
        p = (L - nq + i) if last_positions else i
        logits = []
        for j in range(nk):
            visible = True
            if kv_len is not None and j >= kv_len:
                visible = False
            if causal and j > p:
                visible = False
            if window is not None:
                if window[0] >= 0 and p - j > window[0]:
                    visible = False
                if window[1] >= 0 and j - p > window[1]:
                    visible = False
            if grid is not None:
                cols, nr, nc = grid
                pr, pc = divmod(p, cols)
                jr, jc = divmod(j, cols)
                if abs(pr - jr) >= nr or abs(pc - jc) >= nc:
                    visible = False
            if not visible:
                logits.append(None)
                continue
            dot = 0.0
            for c in range(d):
                dot += q[i][c] * k[j][c]
            x = dot * scale
            if softcap:
                x = softcap * math.tanh(x / softcap)
            if mask is not None:
                x += mask[i][j]
            logits.append(x)
        vis = [x for x in logits if x is not None and x != -math.inf]
        if not vis:
            out.append([0.0] * d)
            lses.append(-math.inf)
            probs.append([0.0] * nk)
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
        probs.append([x / tot for x in w])
    if with_probs:
        return out, lses, probs
    return out, lses
