"""Pure-Python scalar evaluator of the head for tiny dimensions.

Used only as a pin for the fp64 oracle: it is written independently (plain
lists and loops, no numpy, no shared helpers), one scalar at a time, following
the same reading of the pages as the oracle.  Feasible for H, D <= ~64 and a
few dozen rows.
"""
import math


def _f(bits):
    import struct
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _vec(a):
    return [float(x) for x in a]


def _mat(a):
    return [[float(x) for x in row] for row in a]


def _ln(row, w, b, eps):
    n = len(row)
    mu = 0.0
    for x in row:
        mu += x
    mu /= n
    var = 0.0
    for x in row:
        var += (x - mu) * (x - mu)
    var /= n
    r = 1.0 / math.sqrt(var + eps)
    return [(row[i] - mu) * r * w[i] + b[i] for i in range(n)]


def _lin(x, W, b):
    out = []
    for j in range(len(W)):
        acc = 0.0
        for i in range(len(x)):
            acc += W[j][i] * x[i]
        out.append(acc + b[j])
    return out


def _gelu(x):
    return 0.5 * x * (1.0 + math.erf(x / math.sqrt(2.0)))


def _dot(a, b):
    s = 0.0
    for i in range(len(a)):
        s += a[i] * b[i]
    return s


def _cos(a, b):
    na = max(math.sqrt(_dot(a, a)), 1e-8)
    nb = max(math.sqrt(_dot(b, b)), 1e-8)
    return _dot(a, b) / (na * nb)


def _softmax(v):
    m = max(v)
    e = [math.exp(x - m) for x in v]
    s = sum(e)
    return [x / s for x in e]


def _mha(qrows, kvrows, P, pre, heads, nm=("q", "k", "v", "o")):
    Q = [_lin(r, P[f"{pre}.{nm[0]}.w"], P[f"{pre}.{nm[0]}.b"]) for r in qrows]
    K = [_lin(r, P[f"{pre}.{nm[1]}.w"], P[f"{pre}.{nm[1]}.b"]) for r in kvrows]
    V = [_lin(r, P[f"{pre}.{nm[2]}.w"], P[f"{pre}.{nm[2]}.b"]) for r in kvrows]
    D = len(Q[0])
    d = D // heads
    out = []
    for q in Q:
        cat = []
        for j in range(heads):
            sc = []
            for k in K:
                s = 0.0
                for t in range(j * d, (j + 1) * d):
                    s += q[t] * k[t]
                sc.append(s / math.sqrt(d))
            a = _softmax(sc)
            for t in range(j * d, (j + 1) * d):
                acc = 0.0
                for i in range(len(V)):
                    acc += a[i] * V[i][t]
                cat.append(acc)
        out.append(_lin(cat, P[f"{pre}.{nm[3]}.w"], P[f"{pre}.{nm[3]}.b"]))
    return out


def _block(rows, mem, P, pre, heads, eps, xmem=None):
    a = [_ln(r, P[pre + ".ln1.w"], P[pre + ".ln1.b"], eps) for r in rows]
    att = _mha(a, a if mem is None else mem, P, pre, heads)
    rows = [[rows[i][t] + att[i][t] for t in range(len(rows[i]))] for i in range(len(rows))]
    if xmem is not None:   # decoder-layer variant: cross-attention over the memory rows
        a = [_ln(r, P[pre + ".xln.w"], P[pre + ".xln.b"], eps) for r in rows]
        att = _mha(a, xmem, P, pre, heads, ("xq", "xk", "xv", "xo"))
        rows = [[rows[i][t] + att[i][t] for t in range(len(rows[i]))] for i in range(len(rows))]
    out = []
    for r in rows:
        a = _ln(r, P[pre + ".ln2.w"], P[pre + ".ln2.b"], eps)
        h = [_gelu(x) for x in _lin(a, P[pre + ".ffn1.w"], P[pre + ".ffn1.b"])]
        y = _lin(h, P[pre + ".ffn2.w"], P[pre + ".ffn2.b"])
        out.append([r[t] + y[t] for t in range(len(r))])
    return out


def brute_record(weights, head, hidden_bits, q_type, q_span, o_offsets, o_span, o_row_bits):
    """Same contract as the oracle's ``forward_record`` but on bf16 bit patterns."""
    P = {}
    for k, v in weights.items():
        if getattr(v, "dtype", None) is not None and str(v.dtype) == "uint16":
            if v.ndim == 1:
                P[k] = [_f(x) for x in v]
            else:
                P[k] = [[_f(x) for x in row] for row in v]
        else:
            P[k] = [float(x) for x in v]
    eps, heads = head.ln_eps, head.heads
    X = [[_f(x) for x in row] for row in hidden_bits]
    n = len(X)
    XH = [_ln(r, P["ln_in.w"], P["ln_in.b"], eps) for r in X]
    MEM = [_lin(r, P["mem.w"], P["mem.b"]) for r in XH]
    H = len(XH[0])

    def pool(s, e):
        out = [0.0] * H
        for t in range(s, e):
            for i in range(H):
                out[i] += XH[t][i]
        return [v / (e - s) for v in out]

    nq = len(q_type)
    opt_q = []
    for i in range(nq):
        for _ in range(int(o_offsets[i]), int(o_offsets[i + 1])):
            opt_q.append(i)
    qbar = [pool(int(q_span[i][0]), int(q_span[i][1])) for i in range(nq)]
    cbar = [pool(int(s[0]), int(s[1])) for s in o_span]
    g = XH[n - 1]
    ebar = []
    for rows in o_row_bits:
        acc = [0.0] * H
        for row in rows:
            for i in range(H):
                acc[i] += _f(row[i])
        ebar.append([v / len(rows) for v in acc])
    prior = [_cos(ebar[k], [qbar[opt_q[k]][i] + g[i] for i in range(H)]) for k in range(len(o_span))]
    U = []
    for k in range(len(o_span)):
        a = _lin(cbar[k], P["opt_ctx.w"], P["opt_ctx.b"])
        b = _lin(ebar[k], P["opt_lex.w"], P["opt_lex.b"])
        c = _lin(qbar[opt_q[k]], P["q_opt.w"], P["q_opt.b"])
        U.append([a[t] + b[t] + c[t] for t in range(len(a))])
    for r in range(head.routing_layers):
        U = _block(U, MEM, P, f"route.{r}", heads, eps)
    gp = _lin(g, P["glob.w"], P["glob.b"])
    Fv = []
    for i in range(nq):
        o0, o1 = int(o_offsets[i]), int(o_offsets[i + 1])
        sc = [_dot(P["summary.w"], U[k]) + P["summary.b"][0] for k in range(o0, o1)]
        beta = _softmax(sc)
        qv = _lin(qbar[i], P["q_base.w"], P["q_base.b"])
        te = P["type_emb"][int(q_type[i])]
        row = []
        for t in range(len(qv)):
            s = 0.0
            for j, k in enumerate(range(o0, o1)):
                s += beta[j] * U[k][t]
            row.append(qv[t] + s + gp[t] + te[t])
        Fv.append(row)
    xmem = MEM if getattr(head, "field_cross_attention", 0) else None
    for l in range(head.layers):
        Fv = _block(Fv, None, P, f"field.{l}", heads, eps, xmem)
    # logistic gate through tanh (sigma(x) = (1 + tanh(x / 2)) / 2): bounded for every x, -inf included
    gate = 0.5 * (1.0 + math.tanh(0.5 * float(P["gate_logit"][0])))
    lam = P["joint_scale"][0]
    logits = []
    for k in range(len(o_span)):
        f = Fv[opt_q[k]]
        u = U[k]
        z = f + u + [f[t] * u[t] for t in range(len(f))] + [abs(f[t] - u[t]) for t in range(len(f))]
        h = [_gelu(x) for x in _lin(z, P["score.w1"], P["score.b1"])]
        r = _dot(h, P["score.w2"]) + P["score.b2"][0]
        logits.append(prior[k] + gate * (lam * _cos(u, f) + r))
    probs, amax = [], []
    for i in range(nq):
        o0, o1 = int(o_offsets[i]), int(o_offsets[i + 1])
        probs += _softmax(logits[o0:o1])
        best = o0
        for k in range(o0, o1):
            if logits[k] > logits[best]:
                best = k
        amax.append(best - o0)
    return logits, probs, amax
