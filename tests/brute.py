"""Brute-force twins of the oracle for tiny shapes: explicit Python loops over
every index, written from the definitions (rotations as complex numbers,
softmax by hand), sharing no helper with ``oracle/``.  Used only to pin the
vectorised oracle."""
import cmath
import math


def _bf16(x):
    if x == 0.0:
        return 0.0
    m, e = math.frexp(x)
    t = m * 256.0
    r = math.floor(t)
    frac = t - r
    if frac > 0.5 or (frac == 0.5 and r % 2 == 1):
        r += 1
    return math.ldexp(r, e - 8)


def _store(cfg, x):
    return _bf16(x) if cfg.dtype == "bf16" else x


def _rot(vec, p, base):
    d = len(vec)
    out = [0.0] * d
    for j in range(d // 2):
        z = complex(vec[j], vec[j + d // 2]) * cmath.exp(1j * p * base ** (-2.0 * j / d))
        out[j], out[j + d // 2] = z.real, z.imag
    return out


def _matvec(W, x):
    """y[n] = sum_k W[n][k] x[k] with W given as [out][in]."""
    return [sum(float(W[n][k]) * x[k] for k in range(len(x))) for n in range(len(W))]


def _rms(x, gain, eps):
    s = math.sqrt(sum(v * v for v in x) / len(x) + eps)
    return [x[c] / s * float(gain[c]) for c in range(len(x))]


def _kn(cfg, W, l, head):
    """Per-head key RMSNorm when the config asks for QK-norm."""
    return _rms(head, W["k_norm"][l], cfg.rms_eps) if getattr(cfg, "qk_norm", False) else head


def _qn(cfg, W, l, head):
    return _rms(head, W["q_norm"][l], cfg.rms_eps) if getattr(cfg, "qk_norm", False) else head


def inject(cfg, W, x_rows, positions):
    """-> K[l][t][m][e], V[l][t][m][e] as nested lists."""
    L, nkv, d = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
    K = [[None] * len(x_rows) for _ in range(L)]
    V = [[None] * len(x_rows) for _ in range(L)]
    for t, (x, p) in enumerate(zip(x_rows, positions)):
        f = _matvec(W["w_fc"], [float(v) for v in x])
        kv = _matvec(W["w_kv"], f)
        for l in range(L):
            base = l * 2 * nkv * d
            K[l][t] = [[_store(cfg, v) for v in _rot(_kn(cfg, W, l, kv[base + m * d: base + (m + 1) * d]), p,
                                                      cfg.rope_base)]
                       for m in range(nkv)]
            V[l][t] = [[_store(cfg, kv[base + nkv * d + m * d + e]) for e in range(d)] for m in range(nkv)]
    return K, V


def forward(cfg, W, pools, ctx_len, tau, causal=False):
    """LM-head input y[b][i][c] of one draft forward, by explicit loops (causal:
    block token i sees block tokens 0..i only)."""
    H, L = cfg.hidden, cfg.n_layers
    nq, nkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    group = nq // nkv
    out = []
    for b, toks in enumerate(tau):
        B = len(toks)
        T = int(ctx_len[b])
        Kc, Vc = pools[b]
        h = [[float(W["embed"][tok][c]) for c in range(H)] for tok in toks]
        for l in range(L):
            u = [_rms(h[i], W["attn_norm"][l], cfg.rms_eps) for i in range(B)]
            q, k, v = [], [], []
            for i in range(B):
                p = T + i
                qi = _matvec(W["w_q"][l], u[i])
                q.append([_rot(_qn(cfg, W, l, qi[n * d:(n + 1) * d]), p, cfg.rope_base) for n in range(nq)])
                rows = W["w_kv"][l * 2 * nkv * d:(l + 1) * 2 * nkv * d]
                kvi = _matvec(rows, u[i])
                k.append([_rot(_kn(cfg, W, l, kvi[m * d:(m + 1) * d]), p, cfg.rope_base) for m in range(nkv)])
                v.append([kvi[nkv * d + m * d: nkv * d + (m + 1) * d] for m in range(nkv)])
            o = [[None] * nq for _ in range(B)]
            for m in range(nkv):
                for n in range(m * group, (m + 1) * group):
                    for i in range(B):
                        seen = range(i + 1) if causal else range(B)
                        keys = [[float(e) for e in Kc[l][t][m]] for t in range(T)] + [k[j][m] for j in seen]
                        vals = [[float(e) for e in Vc[l][t][m]] for t in range(T)] + [v[j][m] for j in seen]
                        sc = [sum(q[i][n][e] * kk[e] for e in range(d)) / math.sqrt(d) for kk in keys]
                        mx = max(sc)
                        w = [math.exp(s - mx) for s in sc]
                        tot = sum(w)
                        o[i][n] = [sum(w[t] * vals[t][e] for t in range(len(keys))) / tot for e in range(d)]
            for i in range(B):
                flat = [o[i][n][e] for n in range(nq) for e in range(d)]
                ao = _matvec(W["w_o"][l], flat)
                h[i] = [h[i][c] + ao[c] for c in range(H)]
            for i in range(B):
                u2 = _rms(h[i], W["mlp_norm"][l], cfg.rms_eps)
                gt = _matvec(W["w_gate"][l], u2)
                up = _matvec(W["w_up"][l], u2)
                a = [gt[r] / (1.0 + math.exp(-gt[r])) * up[r] for r in range(len(gt))]
                dn = _matvec(W["w_down"][l], a)
                h[i] = [h[i][c] + dn[c] for c in range(H)]
        out.append([[_store(cfg, e) for e in _rms(h[i], W["final_norm"], cfg.rms_eps)] for i in range(B)])
    return out


def greedy_verify(target_logits, draft_tokens):
    acc, outs = [], []
    for zrows, d in zip(target_logits, draft_tokens):
        B = len(d)
        ys = []
        for row in zrows:
            best, bi = -math.inf, -1
            for vi, val in enumerate(row):
                if val > best:
                    best, bi = val, vi
            ys.append(bi)
        a = B
        for i in range(B):
            if ys[i] != d[i]:
                a = i
                break
        acc.append(a)
        outs.append(list(d[:a]) + [ys[a]] + [-1] * (B - a))
    return acc, outs
