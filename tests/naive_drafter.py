"""A second, naive oracle of the draft step: scalar Python loops, tiny shapes.

TEST INFRASTRUCTURE, written separately from oracle/dlite_oracle.py and
sharing nothing with it: every value is a Python float, every sum an explicit
loop, every matrix a nested list.  It exists to pin the composition of the
draft step (which slot sits at which local position, which rows query, how the
rotary pairs are formed, how the heads group, where each norm and residual
goes) on shapes small enough for scalar loops (D = 8, V = 16, r = 4, K = 3,
m = 2).  The numpy oracle must agree with it to 1e-12.

Sources (page title and section):
  "DLite 完全拆解" walkthrough: the depth-embedded, normalised features kept as
  separate sequence slots ("历史并没有消失，而是由目标模型编码", "沿序列维拼接，保留各层
  的独立身份"); Figure 3's local coordinates, every feature slot and the anchor
  at local position 0 and the placeholders at 1, 2, 3, ... ("局部位置编码切断草稿端
  的全局位置增长"); queries from the anchor and placeholders, keys and values from
  every slot, no causal mask inside the block ("锚点是已经确定、尚待目标前向处理的
  输入", "本轮临时 K/V 仍然需要计算"); a low-rank state over the block positions
  followed by one vocabulary projection ("轻量顺序头：只补块内依赖",
  "避免的是昂贵的中间词表投影"); greedy choice at temperature 0.
The same readings as the main oracle fill what the pages leave open: RMSNorm
with a gain, rotate-half rotary pairs with frequency theta^(-2i/d_h), pre-norm
grouped attention and SwiGLU layers without biases, a final RMSNorm, the fixed
recurrence s_k = s_{k-1} + W_up silu(W_down [h_k; s_{k-1}]) from s_0 = 0, and
ties to the lowest vocabulary index.
"""
import math


def _mat(a):
    """Nested lists of Python floats from any 1-D / 2-D array-like."""
    try:
        return [[float(v) for v in row] for row in a]
    except TypeError:
        return [float(v) for v in a]


def _rmsnorm_row(x, gain, eps):
    ss = 0.0
    for v in x:
        ss += v * v
    inv = 1.0 / math.sqrt(ss / len(x) + eps)
    return [gain[i] * x[i] * inv for i in range(len(x))]


def _matvec(W, x):
    out = []
    for row in W:
        acc = 0.0
        for j in range(len(x)):
            acc += row[j] * x[j]
        out.append(acc)
    return out


def _silu(t):
    return t / (1.0 + math.exp(-t))


def _position(slot, m, G=1, n_valid=1):
    """Local position of a slot.  Figure 3 (G = 1): features (slots 0..m-1)
    and the anchor (slot m) at 0, placeholder k (slot m + k) at k.  With a
    token group of G slots (n_valid real, padded at the front), the origin is
    the first real group token: group slot j at j - (G - n_valid), the
    features at the anchor's position n_valid - 1, placeholder k at
    n_valid - 1 + k."""
    pad = G - n_valid
    if slot < m:
        return n_valid - 1
    if slot < m + G:
        j = slot - m
        return j - pad if j >= pad else 0
    return n_valid - 1 + (slot - m - G + 1)


def _is_key(slot, m, G=1, n_valid=1):
    """Padding slots of the token group are not keys."""
    return not (m <= slot < m + G - n_valid)


def _rotate(vec, p, theta):
    """Rotate each pair (i, i + d/2) of one head vector by p * theta^(-2i/d)."""
    d = len(vec)
    half = d // 2
    out = [0.0] * d
    for i in range(half):
        ang = p * theta ** (-2.0 * i / d)
        c, s = math.cos(ang), math.sin(ang)
        out[i] = vec[i] * c - vec[i + half] * s
        out[i + half] = vec[i] * s + vec[i + half] * c
    return out


def _layer(ctx, x, lw, dims, G=1, n_valid=1):
    """One pre-norm layer for one request: ctx [m][D] (keys/values only),
    x [G+K][D] local residual rows (anchor or token group, placeholders)."""
    m = len(ctx)
    n_q, n_kv, dh = dims.n_q, dims.n_kv, dims.d_h
    eps, theta = dims.rms_eps, dims.rope_theta
    per_kv = n_q // n_kv            # query heads per key/value head
    slots = list(ctx) + list(x)
    S = len(slots)
    wqkv = lw["wqkv"]
    q_rows = wqkv[: n_q * dh]
    k_rows = wqkv[n_q * dh: (n_q + n_kv) * dh]
    v_rows = wqkv[(n_q + n_kv) * dh:]
    normed = [_rmsnorm_row(sl, lw["attn_norm"], eps) for sl in slots]
    # keys and values of every slot, rotated keys at the slot's local position
    keys, vals = [], []
    for s in range(S):
        kf = _matvec(k_rows, normed[s])
        vf = _matvec(v_rows, normed[s])
        keys.append([_rotate(kf[g * dh:(g + 1) * dh], _position(s, m, G, n_valid), theta)
                     for g in range(n_kv)])
        vals.append([vf[g * dh:(g + 1) * dh] for g in range(n_kv)])
    new_x = []
    for j in range(len(x)):
        slot = m + j
        qf = _matvec(q_rows, normed[slot])
        attn = []
        for h in range(n_q):
            qh = _rotate(qf[h * dh:(h + 1) * dh], _position(slot, m, G, n_valid), theta)
            g = h // per_kv
            scores = []
            for s in range(S):
                dot = 0.0
                for t in range(dh):
                    dot += qh[t] * keys[s][g][t]
                scores.append(dot / math.sqrt(dh))
            mx = max(scores[s] for s in range(S) if _is_key(s, m, G, n_valid))
            ex = [math.exp(scores[s] - mx) if _is_key(s, m, G, n_valid) else 0.0 for s in range(S)]
            tot = sum(ex)
            for t in range(dh):
                acc = 0.0
                for s in range(S):
                    acc += ex[s] / tot * vals[s][g][t]
                attn.append(acc)
        o = _matvec(lw["wo"], attn)
        r1 = [x[j][i] + o[i] for i in range(len(o))]
        n2 = _rmsnorm_row(r1, lw["ffn_norm"], eps)
        F = len(lw["w_down"][0])
        gu = _matvec(lw["w_gate_up"], n2)
        act = [_silu(gu[f]) * gu[F + f] for f in range(F)]
        down = _matvec(lw["w_down"], act)
        new_x.append([r1[i] + down[i] for i in range(len(r1))])
    return new_x


def naive_draft(dims, weights, H, anchor_rows, group_rows=None, group_valid=None):
    """The whole draft step with scalar loops.

    weights: fp64 arrays keyed as the main oracle's (layers list); H [B][m][D];
    anchor_rows [B][D]; or a local token group: group_rows [B][G][D] with
    group_valid [B] real tokens at the end of each group.  Returns dict of
    nested lists: z, x_layers, h, s, logits, cand.
    """
    B, m, K = dims.B, dims.m, dims.K
    eps = dims.rms_eps
    dep = _mat(weights["depth_emb"])
    fgain = _mat(weights["feat_norm"])
    ph = _mat(weights["ph_emb"])
    layers = [{k: _mat(v) for k, v in lw.items()} for lw in weights["layers"]]
    fin = _mat(weights["final_norm"])
    wd = _mat(weights["seq_w_down"])
    wu = _mat(weights["seq_w_up"])
    lm = _mat(weights["lm_head"])
    r = len(wu)
    out = dict(z=[], x_layers=[[] for _ in layers], h=[], s=[], logits=[], cand=[])
    for b in range(B):
        ctx = []
        for l in range(m):
            row = [float(H[b][l][i]) + dep[l][i] for i in range(len(dep[l]))]
            ctx.append(_rmsnorm_row(row, fgain, eps))
        out["z"].append(ctx)
        if group_rows is None:
            G, nv = 1, 1
            lead = [[float(v) for v in anchor_rows[b]]]
        else:
            G, nv = len(group_rows[b]), int(group_valid[b])
            lead = [[float(v) for v in group_rows[b][j]] if j >= G - nv else [0.0] * len(ph)
                    for j in range(G)]
        x = lead + [list(ph) for _ in range(K)]
        for li, lw in enumerate(layers):
            x = _layer(ctx, x, lw, dims, G, nv)
            out["x_layers"][li].append([list(row) for row in x])
        hs = [_rmsnorm_row(x[G + k], fin, eps) for k in range(K)]
        out["h"].append(hs)
        state = [0.0] * r
        states, logits, cands = [], [], []
        for k in range(K):
            t = _matvec(wd, hs[k] + state)
            upd = _matvec(wu, [_silu(v) for v in t])
            state = [state[i] + upd[i] for i in range(r)]
            states.append(list(state))
            lg = _matvec(lm, state)
            best = 0
            for v in range(1, len(lg)):
                if lg[v] > lg[best]:
                    best = v
            logits.append(lg)
            cands.append(best)
        out["s"].append(states)
        out["logits"].append(logits)
        out["cand"].append(cands)
    return out
