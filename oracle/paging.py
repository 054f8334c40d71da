"""Monarch-style hot/cold paging of one (sequence, layer) (oracle).

Test infrastructure (see the package docstring).  Deliberately a brute-force
simulator over explicit Python lists.

"Monarch v3: Paginacion KV Inspirada en NES" (openclawradar.com), section
"Como funciona": a hot region of recent tokens at full precision, a cold
region of compressed tokens, sliding-window eviction of old tokens to cold,
and attention-weighted promotion back to hot with a sticky mechanism against
thrashing; section "Bucle de Decodificacion Simplificado": attend, move
high-attention cold tokens to hot for the next step, evict the oldest hot
tokens to cold when the window overflows; section "Como probarlo": the
promotion threshold (0.15) and sticky threshold (3) flags.

Readings taken where the page is silent:

* Step order: append (then evict while more than W entries are hot) ->
  attend -> promote.
* Eviction is FIFO by time of entry into the hot window (a ring of the W most
  recent entries); promoted tokens enter as the newest entries.
* An evicted NEW token is quantised into the next cold slot (slots are
  append-only).  An evicted PROMOTED token is not re-quantised: its cold code
  was kept (tombstoned) while it was hot, and eviction revives it.
* Promotion statistic of a live cold slot c: P_c = max over the layer's query
  heads of its full-softmax probability (hot and cold tokens together).
* Sticky counter: cnt_c += 1 on a step with P_c >= tau, else reset to 0;
  reset after promotion and on re-eviction.  A slot is promoted on the step
  its counter reaches ``sticky``.  All slots promoted in one step enter the
  hot window in order of P_c descending, ties to the lower slot.
* A promoted token's hot key and value are the fp16 (round-to-nearest-even)
  dequantisation of its codes, QJL term included (for values only when the
  value QJL term is on).
* tau > 1 disables promotion (window-only paging, the fallback the page
  names for models whose attention cannot be read).
"""

import numpy as np

from . import attention as _att
from . import codec as _codec


class HotEntry:
    __slots__ = ("slot", "k", "v", "pos")

    def __init__(self, slot, k, v, pos):
        self.slot = slot  # None for NEW, else the cold slot it was promoted from
        self.k = k  # [H_kv, d] fp16
        self.v = v
        self.pos = pos  # token position (bookkeeping only)


class SeqLayerCache:
    """Hot/cold cache of one (sequence, layer)."""

    def __init__(self, n_kv_heads, d, window, fmt, pi, s_full, tau=2.0, sticky=3, v_qjl=True):
        self.hkv, self.d, self.W = n_kv_heads, d, window
        self.fmt, self.pi, self.s = fmt, pi, s_full
        self.tau, self.sticky, self.v_qjl = tau, sticky, v_qjl
        self.hot = []  # FIFO, oldest first
        self.cold_k = [[] for _ in range(n_kv_heads)]  # per kv-head list of single-vector code dicts
        self.cold_v = [[] for _ in range(n_kv_heads)]
        # boundary-band masks per slot (which fields an fp32 encoder may decide otherwise)
        self.band_k = [[] for _ in range(n_kv_heads)]
        self.band_v = [[] for _ in range(n_kv_heads)]
        self.cold_pos = []
        self.live = []
        self.cnt = []
        self.n_tokens = 0
        self.n_evicted = 0
        self.n_promoted = 0
        self.near_tau = []  # (step, slot, P) with |P - tau| <= 2e-3 * tau
        self.step = 0

    # -- eviction -----------------------------------------------------------
    def _evict_oldest(self, pending):
        e = self.hot.pop(0)
        self.n_evicted += 1
        if e.slot is None:
            pending.append(e)
        else:
            self.live[e.slot] = True
            self.cnt[e.slot] = 0

    def _flush(self, pending):
        if not pending:
            return
        for kv in range(self.hkv):
            ks = np.stack([e.k[kv] for e in pending])
            vs = np.stack([e.v[kv] for e in pending])
            ck = _codec.quantize(ks, self.pi, self.s, self.fmt)
            cv = _codec.quantize(vs, self.pi, self.s, self.fmt)
            bk = _codec.boundary_band(ck, self.s, self.fmt)
            bv = _codec.boundary_band(cv, self.s, self.fmt)
            for i in range(len(pending)):
                self.cold_k[kv].append(_slice_codes(ck, i))
                self.cold_v[kv].append(_slice_codes(cv, i))
                self.band_k[kv].append({key: bk[key][i] for key in _BAND_KEYS})
                self.band_v[kv].append({key: bv[key][i] for key in _BAND_KEYS})
        for e in pending:
            self.cold_pos.append(e.pos)
            self.live.append(True)
            self.cnt.append(0)

    def append(self, k16, v16):
        """Append n >= 0 tokens (k16, v16: [n, H_kv, d] fp16), then evict to W."""
        k16 = np.asarray(k16, dtype=np.float16)
        v16 = np.asarray(v16, dtype=np.float16)
        pending = []
        for t in range(k16.shape[0]):
            self.hot.append(HotEntry(None, k16[t].copy(), v16[t].copy(), self.n_tokens))
            self.n_tokens += 1
        # FIFO: evicting after all pushes pops the same entries in the same
        # order as evicting after each push; an empty append still trims
        # promoted overflow back to the window
        while len(self.hot) > self.W:
            self._evict_oldest(pending)
        self._flush(pending)

    def evict(self, target):
        """Evict without an append: oldest first while more than target
        entries are hot (the same FIFO step as append's)."""
        pending = []
        while len(self.hot) > target:
            self._evict_oldest(pending)
        self._flush(pending)

    # -- attention ----------------------------------------------------------
    def cold_codes(self, kv, which="k"):
        lst = (self.cold_k if which == "k" else self.cold_v)[kv]
        return _stack_codes(lst, self.d, self.fmt)

    def hot_arrays(self):
        if not self.hot:
            z = np.zeros((self.hkv, 0, self.d), dtype=np.float16)
            return z, z
        hk = np.stack([e.k for e in self.hot], axis=1)
        hv = np.stack([e.v for e in self.hot], axis=1)
        return hk, hv

    def attend(self, q16, gate=np.inf):
        """One attention step (gate: the hot-first threshold, see
        attention.decode_attention; +inf scores the cold slots always)."""
        hk, hv = self.hot_arrays()
        ck = [self.cold_codes(kv, "k") for kv in range(self.hkv)]
        cv = [self.cold_codes(kv, "v") for kv in range(self.hkv)]
        res = _att.decode_attention(q16, hk, hv, ck, cv, np.array(self.live, dtype=bool),
                                    self.pi, self.s, self.fmt, self.v_qjl, gate=gate)
        n_cold = len(self.live)
        res["P"] = res["p_cold"].max(axis=0) if n_cold else np.zeros(0)
        self.step += 1
        return res

    # -- promotion ----------------------------------------------------------
    def promote(self, P):
        """Sticky counters from this step's P, then promote the qualifiers."""
        if self.tau > 1.0:
            return []
        hits = []
        for c in range(len(self.live)):
            if not self.live[c]:
                continue
            if abs(P[c] - self.tau) <= 2e-3 * self.tau:
                self.near_tau.append((self.step, c, float(P[c])))
            if P[c] >= self.tau:
                self.cnt[c] += 1
            else:
                self.cnt[c] = 0
            if self.cnt[c] >= self.sticky:
                hits.append(c)
        hits.sort(key=lambda c: (-P[c], c))
        for c in hits:
            kk = np.zeros((self.hkv, self.d), dtype=np.float16)
            vv = np.zeros((self.hkv, self.d), dtype=np.float16)
            for kv in range(self.hkv):
                ck = _stack_codes([self.cold_k[kv][c]], self.d, self.fmt)
                cv = _stack_codes([self.cold_v[kv][c]], self.d, self.fmt)
                kk[kv] = _codec.to_f16(_codec.dequantize(ck, self.pi, self.s, self.fmt, qjl=True)[0])
                vv[kv] = _codec.to_f16(_codec.dequantize(cv, self.pi, self.s, self.fmt, qjl=self.v_qjl)[0])
            self.hot.append(HotEntry(c, kk, vv, self.cold_pos[c]))
            self.live[c] = False
            self.cnt[c] = 0
            self.n_promoted += 1
        return hits

    # -- views for tests ----------------------------------------------------
    def hot_tags(self):
        """FIFO list of tags: -1 for NEW, else the cold slot."""
        return [-1 if e.slot is None else e.slot for e in self.hot]

    def hot_positions(self):
        return [e.pos for e in self.hot]


_CODE_KEYS = ("a", "b", "R16", "rho16", "signs")
_BAND_KEYS = ("pair", "R", "rho", "sign", "vector")


def _slice_codes(codes, i):
    return {k: codes[k][i] for k in _CODE_KEYS}


def _stack_codes(lst, d, fmt):
    if not lst:
        p = d // 2
        return dict(a=np.zeros((0, p), np.int64), b=np.zeros((0, p), np.int64),
                    R16=np.zeros(0, np.float16), rho16=np.zeros(0, np.float16),
                    signs=np.zeros((0, fmt.m), bool))
    return {k: np.stack([c[k] for c in lst]) for k in _CODE_KEYS}
