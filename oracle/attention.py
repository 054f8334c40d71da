"""Decode attention read directly from the compressed cache (oracle, fp64).

Test infrastructure (see the package docstring).

"TurboQuant: optimizacion de memoria para KV caches" (kerneldigest.dev),
step six of its quantisation flow: attention logits are computed from the
compressed cache; section "Arquitectura del Sistema": QJL keeps the attention
score accurate.  The logit of a cold key follows the polar code plus the QJL
estimator of the residual inner product:

    l_j = [ <q', y_hat_j> + sqrt(pi/2)/m * rho_j * <S_m q', sigma_j> ] / sqrt(d)

with q' = Pi q.  Algebraically l_j = <q, x_hat_j> / sqrt(d) where x_hat_j is
the QJL-inclusive dequantised key; the tests check that identity.

Readings taken here: logits are scaled by 1/sqrt(d) with no mask (the decode
step sees every live token, including the one just appended); grouped-query
attention maps q-head h to kv-head h // (H_q / H_kv); hot keys and values are
the fp16 entries of the hot window, read exactly; cold values are dequantised
(with the QJL term unless disabled); the output is accumulated in fp64 and
reported as fp32.

The hot-first loop of "Monarch v3" (section "Bucle de Decodificacion
Simplificado") scores the hot window and then the cold pages; here both
regions enter one softmax over all live tokens.  Its gate (the cold pages are
scored only when the best hot score falls below a threshold) is the optional
``gate`` argument of decode_attention; the default (+inf) scores cold always.
"""

import numpy as np

from .codec import SQRT_HALF_PI, Format


def rotate_query(q: np.ndarray, pi: np.ndarray) -> np.ndarray:
    """q' = Pi q for each row of q [H, d]."""
    return np.asarray(q, dtype=np.float64) @ pi.T


def cold_logits(q: np.ndarray, codes: dict, pi: np.ndarray, s_full: np.ndarray, fmt: Format) -> np.ndarray:
    """Code-domain logits [H, N] of query rows q [H, d] against N coded keys.

    Polar term through a per-pair table T_i[b] = q'_{2i} cos(phi_b) +
    q'_{2i+1} sin(phi_b) scaled by a_i * R / (L_r - 1); QJL term through
    <S_m q', sigma>.
    """
    q = np.asarray(q, dtype=np.float64)
    h, d = q.shape
    qr = rotate_query(q, pi)
    phi = -np.pi + 2.0 * np.pi * np.arange(fmt.n_angle) / fmt.n_angle
    # table[h, i, b]
    tab = qr[:, 0::2, None] * np.cos(phi)[None, None, :] + qr[:, 1::2, None] * np.sin(phi)[None, None, :]
    a, b = codes["a"], codes["b"]
    n, p = a.shape
    R = codes["R16"].astype(np.float64)
    idx_i = np.arange(p)[None, :]
    polar = np.empty((h, n))
    for hh in range(h):
        polar[hh] = (a * tab[hh][idx_i, b]).sum(axis=1) * R / (fmt.n_radius - 1)
    sq = qr @ s_full[: fmt.m].T  # [H, m]
    sigma = 2.0 * codes["signs"].astype(np.float64) - 1.0  # [N, m]
    rho = codes["rho16"].astype(np.float64)
    qjl = (SQRT_HALF_PI / fmt.m) * rho[None, :] * (sq @ sigma.T)
    return (polar + qjl) / np.sqrt(d)


def hot_logits(q: np.ndarray, k16: np.ndarray) -> np.ndarray:
    """Logits [H, n] against fp16 keys k16 [n, d] held exactly."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k16, dtype=np.float16).astype(np.float64)
    return (q @ k.T) / np.sqrt(q.shape[1])


def softmax(logits: np.ndarray) -> np.ndarray:
    """Row-wise softmax; -inf entries get probability 0."""
    m = np.max(logits, axis=-1, keepdims=True)
    w = np.exp(logits - m)
    return w / w.sum(axis=-1, keepdims=True)


def decode_attention(q16, hot_k, hot_v, cold_k, cold_v, live, pi, s_full, fmt: Format, v_qjl: bool = True,
                     gate: float = np.inf):
    """One decode step of one (sequence, layer) over hot and cold tokens.

    q16: [H_q, d] fp16 queries.  hot_k, hot_v: [H_kv, n_hot, d] fp16.
    cold_k, cold_v: lists (one per kv-head) of code dicts over n_cold slots.
    live: [n_cold] bool (False where a slot is tombstoned because its token
    is currently promoted to the hot window).
    gate: the hot-first gate of "Monarch v3", section "Bucle de
    Decodificacion Simplificado" (score the cold pages only if the best hot
    score is below a threshold).  Readings: the score is the scaled logit
    <q, k>/sqrt(d); a cold page holds one kv head's tokens, so the decision is
    per kv head -- its cold slots are scored when any query head of its group
    has its best hot logit below ``gate`` (or the window is empty), and
    otherwise every head of the group attends over the hot tokens only.
    gate = +inf: cold is always scored (the plain decode step).
    Returns dict(out [H_q, d] fp64, logits_hot [H_q, n_hot],
    logits_cold [H_q, n_cold] (-inf where not live or not scored), p_hot,
    p_cold, gated [H_kv] (True where the group skipped its cold slots),
    gate_margin [H_kv] (min over the group's heads of the best hot logit,
    minus gate; -inf without hot tokens)).
    """
    from .codec import dequantize

    q = np.asarray(q16, dtype=np.float16).astype(np.float64)
    hq, d = q.shape
    hkv = hot_k.shape[0]
    g = hq // hkv
    n_hot = hot_k.shape[1]
    n_cold = len(live)
    out = np.zeros((hq, d))
    lh = np.full((hq, n_hot), -np.inf)
    lc = np.full((hq, n_cold), -np.inf)
    ph = np.zeros((hq, n_hot))
    pc = np.zeros((hq, n_cold))
    gated = np.zeros(hkv, dtype=bool)
    margin = np.full(hkv, -np.inf)
    for kv in range(hkv):
        rows = slice(kv * g, (kv + 1) * g)
        qq = q[rows]
        l_hot = hot_logits(qq, hot_k[kv]) if n_hot else np.zeros((g, 0))
        if n_hot:
            margin[kv] = l_hot.max(axis=1).min() - gate
        gated[kv] = n_cold > 0 and n_hot > 0 and margin[kv] >= 0.0
        if n_cold and not gated[kv]:
            l_cold = cold_logits(qq, cold_k[kv], pi, s_full, fmt)
            l_cold = np.where(np.asarray(live)[None, :], l_cold, -np.inf)
        else:
            l_cold = np.full((g, n_cold), -np.inf)
        allv = np.concatenate([l_hot, l_cold], axis=1)
        p = softmax(allv)
        p_hot, p_cold = p[:, :n_hot], p[:, n_hot:]
        o = p_hot @ hot_v[kv].astype(np.float64) if n_hot else np.zeros((g, d))
        if n_cold and not gated[kv]:
            vh = dequantize(cold_v[kv], pi, s_full, fmt, qjl=v_qjl)
            o = o + p_cold @ vh
        out[rows] = o
        lh[rows], lc[rows], ph[rows], pc[rows] = l_hot, l_cold, p_hot, p_cold
    return dict(out=out, logits_hot=lh, logits_cold=lc, p_hot=ph, p_cold=pc, gated=gated, gate_margin=margin)


def multi_query_attention(q16, hot_k, hot_v, cold_k, cold_v, live, pi, s_full, fmt: Format, n_new: int,
                          v_qjl: bool = True):
    """Attention of the n_new newest tokens' queries (a prefill chunk, or
    draft tokens being verified) over one (sequence, layer) after they were
    appended: query j (0 = oldest of the chunk) sees every live cold slot and
    the hot entries up to its own token, i.e. the first n_hot - n_new + j + 1
    entries of the FIFO (the chunk's tokens are its newest n_new entries).

    q16: [n_new, H_q, d].  Returns out [n_new, H_q, d]."""
    q16 = np.asarray(q16, dtype=np.float16)
    n_hot = hot_k.shape[1]
    if n_new > n_hot:
        raise ValueError("the chunk's tokens must all be in the hot window")
    out = np.zeros(q16.shape)
    for j in range(n_new):
        vis = n_hot - n_new + j + 1
        res = decode_attention(q16[j], hot_k[:, :vis], hot_v[:, :vis], cold_k, cold_v, live, pi, s_full, fmt,
                               v_qjl)
        out[j] = res["out"]
    return out


def exact_attention(q16, k16, v16):
    """Textbook softmax attention of fp16 queries [H_q, d] over fp16 keys and
    values [H_kv, n, d] (grouped-query), fp64.  The uncompressed baseline."""
    q = np.asarray(q16, dtype=np.float16).astype(np.float64)
    hq, d = q.shape
    hkv = k16.shape[0]
    g = hq // hkv
    out = np.zeros((hq, d))
    for kv in range(hkv):
        rows = slice(kv * g, (kv + 1) * g)
        p = softmax(hot_logits(q[rows], k16[kv]))
        out[rows] = p @ np.asarray(v16[kv], dtype=np.float16).astype(np.float64)
    return out


def partial_state(logits: np.ndarray, values: np.ndarray):
    """Per-chunk softmax state (max, sum of exp, unnormalised accumulator)."""
    m = np.max(logits, axis=-1)
    w = np.exp(logits - m[..., None])
    return m, w.sum(axis=-1), w @ values


def merge_partials(states):
    """Merge per-chunk (max, sum, acc) states into the normalised output."""
    ms = np.stack([s[0] for s in states])
    mg = ms.max(axis=0)
    scale = np.exp(ms - mg[None])
    lsum = sum(s[1] * sc for s, sc in zip(states, scale))
    acc = sum(s[2] * sc[..., None] for s, sc in zip(states, scale))
    return acc / lsum[..., None]
