"""CPU interpreter of the megakernel's per-CU instruction streams (a test of
the schedule, never a reference for the GPU results).

It runs the task streams mk_create builds -- the same descriptors the kernel
reads, exported by mk_plan_streams -- in float64 on small models, in a random
interleaving of the CUs.  Each task phase waits, as on the device, until the
data it polls has been written: a stage's input words and their sums of
squares, the residual of O / down, the split-K partial slots of a group's
piece 0 or of a K-split finish task, the attention partials of a segment's
finisher.  The attention partition is derived from seq_lens exactly as the
device cuts it.  Any interleaving must

  * finish (no phase waits on data that is never written: no deadlock),
  * write every output element exactly once and read every partial slot
    exactly once (no lost or double work),
  * give bit-identical results (no result depends on the order the CUs ran
    in: no race).

The tile arithmetic itself is plain float64 numpy, so the interpreter's
results also match the float64 oracle to rounding order.
"""
from __future__ import annotations

import math

import numpy as np

from decode_megakernel_amd import binding

QKV, ATTN, O, GU, DOWN, LM, EMB = range(7)
T_EMBED, T_GEMV, T_ATTN, T_FIN = 1, 2, 3, 4
F_PUBLISH = 2


class Deadlock(AssertionError):
    pass


class Interp:
    def __init__(self, shape, W, kv_k, kv_v, tokens, positions, n_cu, max_batch=16, attn_pad=None, min_rows=32):
        """W: oracle.Weights (float64 on use); kv_k / kv_v: float64 [L][b][nkv][>= max pos][hd]
        prompt rows; tokens / positions: per sequence."""
        self.sh, self.W = shape, W
        self.b = len(tokens)
        self.tok, self.pos = list(tokens), list(positions)
        self.n_cu = n_cu
        self.streams, self.amap = binding.plan_streams(shape, self.b, n_cu, max_batch=max_batch,
                                                       max_seq=max(positions) + 2)
        sh = shape
        L, d, b, hd = sh.n_layers, sh.hidden, self.b, sh.head_dim
        self.nkv, self.G = sh.n_kv_heads, sh.group
        self.qdim, self.kvdim = sh.q_dim, sh.kv_dim
        self.nqkv = self.qdim + 2 * self.kvdim
        self.K, self.V = kv_k, kv_v
        self.attn_pad = (256 << 10) // (4 * hd) if attn_pad is None else attn_pad
        self.min_rows = min_rows
        nan = lambda *s: np.full(s, np.nan)
        self.buf = {
            "hres": nan(L + 1, b, d), "xattn": nan(L + 1, b, d), "ssattn": nan(L + 1, b, d // 16),
            "hmid": nan(L, b, d), "xmlp": nan(L, b, d), "ssmlp": nan(L, b, d // 16),
            "qkv": nan(L, b, self.nqkv), "aout": nan(L, b, self.qdim), "act": nan(L, b, sh.intermediate),
            "logits": nan(b, sh.vocab), "knew": nan(L, b, self.nkv, hd), "vnew": nan(L, b, self.nkv, hd),
        }
        self.slots = {}        # split-K / K-split partial tiles and attention partials: key -> value
        self.slot_writes = set()
        # per-CU program: list of (ready(), run()) phases
        self.prog = [self._program(c) for c in range(n_cu)]

    # ---------------------------------------------------------------- data
    def _w(self, name):
        return self.W.get(name)

    def _stage_rows(self, st):
        sh = self.sh
        return {QKV: self.nqkv, O: sh.hidden, GU: 2 * sh.intermediate, DOWN: sh.hidden, LM: sh.vocab}[st]

    def _stage_in(self, st, l):
        return {QKV: ("xattn", l), O: ("aout", l), GU: ("xmlp", l), DOWN: ("act", l), LM: ("xattn", self.sh.n_layers)}[st]

    def _stage_ss(self, st, l):
        return {QKV: ("ssattn", l), GU: ("ssmlp", l), LM: ("ssattn", self.sh.n_layers)}.get(st)

    def _weight_rows(self, st, l, rows):
        """Weight rows of the stage's logical rows (QKV: q|k|v stacked; gate/up:
        16-row logical tiles of 8 gate rows then the same 8 up rows)."""
        p = f"model.layers.{l}."
        cache = self.__dict__.setdefault("_wcache", {})
        if st == QKV:
            if (st, l) not in cache:
                cache[(st, l)] = np.concatenate([self._w(p + "self_attn.q_proj.weight"),
                                                 self._w(p + "self_attn.k_proj.weight"),
                                                 self._w(p + "self_attn.v_proj.weight")], 0)
            return cache[(st, l)][rows]
        if st == O:
            return self._w(p + "self_attn.o_proj.weight")[rows]
        if st == GU:
            if (st, l) not in cache:
                g, u = self._w(p + "mlp.gate_proj.weight"), self._w(p + "mlp.up_proj.weight")
                I = g.shape[0]
                lr = np.arange(2 * I)
                j = lr & 15
                src = 8 * (lr >> 4) + (j & 7)
                cache[(st, l)] = np.where((j < 8)[:, None], g[src], u[src])
            return cache[(st, l)][rows]
        if st == DOWN:
            return self._w(p + "mlp.down_proj.weight")[rows]
        name = "model.embed_tokens.weight" if self.sh.tied_embeddings else "lm_head.weight"
        return self._w(name)[rows]

    def _written(self, key, l, n, lo, hi):
        a = self.buf[key][l] if l is not None else self.buf[key]
        return not np.isnan(a[n, lo:hi]).any()

    def _write(self, key, idx, val):
        a = self.buf[key]
        cur = a[idx]
        assert np.isnan(cur).all(), f"{key}{idx} written twice"
        a[idx] = val

    def _take_slot(self, key):
        assert key in self.slots, f"slot {key} read before written (or twice)"
        return self.slots.pop(key)

    def _put_slot(self, key, val):
        assert key not in self.slots and key not in self.slot_writes, f"slot {key} written twice"
        self.slot_writes.add(key)
        self.slots[key] = val

    def _rms(self, st, l, n):
        key, ll = self._stage_ss(st, l)
        return 1.0 / math.sqrt(self.buf[key][ll, n].sum() / self.sh.hidden + self.sh.rms_eps)

    # ------------------------------------------------------------ epilogues
    def _epilogue(self, st, l, rows, val):
        """val [b][len(rows)]: the sums of the tile; rows: logical rows (< M)."""
        sh, b = self.sh, self.b
        rows = np.asarray(rows)
        if st == QKV:
            for n in range(b):
                self._write("qkv", (l, n, rows), self._rms(st, l, n) * val[n])
        elif st in (O, DOWN):
            hin = self.buf["hres"][l] if st == O else self.buf["hmid"][l]
            nw = (self._w(f"model.layers.{l}.post_attention_layernorm.weight") if st == O else
                  self._w(f"model.layers.{l + 1}.input_layernorm.weight") if l + 1 < sh.n_layers else
                  self._w("model.norm.weight"))
            ko, kx, ks, lo = ("hmid", "xmlp", "ssmlp", l) if st == O else ("hres", "xattn", "ssattn", l + 1)
            for n in range(b):
                h = hin[n, rows] + val[n]
                self._write(ko, (lo, n, rows), h)
                self._write(kx, (lo, n, rows), h * nw[rows])
                for t in np.unique(rows // 16):
                    m = rows // 16 == t
                    assert m.sum() == 16
                    self._write(ks, (lo, n, t), float(np.sum(h[m] ** 2)))
        elif st == GU:
            for n in range(b):
                r = self._rms(st, l, n)
                for t in np.unique(rows >> 4):
                    m = (rows >> 4) == t
                    rr = rows[m]
                    vv = val[n][m]
                    g = r * vv[(rr & 15) < 8]
                    u = r * vv[(rr & 15) >= 8]
                    self._write("act", (l, n, 8 * t + np.arange(8)), g / (1.0 + np.exp(-g)) * u)
        else:
            for n in range(b):
                self._write("logits", (n, rows), self._rms(st, l, n) * val[n])

    # ----------------------------------------------------------- programs
    def _gemv_phases(self, t):
        st, l = t["stage"], t["layer"]
        M = self._stage_rows(st)
        key, ll = self._stage_in(st, l)
        k0, k1 = t["k0"], t["k1"]
        subs = list(range(t["row0"] // 16, t["row0"] // 16 + t["nsub"]))
        publish = bool(t["flags"] & F_PUBLISH)
        ss = self._stage_ss(st, l)

        def inputs_ready():
            if not all(self._written(key, ll, n, k0, k1) for n in range(self.b)):
                return False
            if ss and not publish:
                if np.isnan(self.buf[ss[0]][ss[1]]).any():
                    return False
            return True

        def partial(u):
            rows = [r for r in range(16 * u, 16 * u + 16) if r < M]
            Wt = self._weight_rows(st, l, rows)[:, k0:k1]
            x = self.buf[key][ll][:, k0:k1]
            return rows, x @ Wt.T  # [b][rows]

        def resid_ready(rows):
            if st not in (O, DOWN):
                return True
            hin = "hres" if st == O else "hmid"
            return all(self._written(hin, l, n, rows[0], rows[-1] + 1) for n in range(self.b))

        if publish:
            def run():
                for u in subs:
                    _, v = partial(u)
                    self._put_slot(("ks", l, t["part_slot"] + u * t["nks"] + t["ks"]), v)
            return [(inputs_ready, run)]
        if t["nks"] == 1:
            all_rows = [r for u in subs for r in range(16 * u, 16 * u + 16) if r < M]

            def run1():
                for u in subs:
                    rows, v = partial(u)
                    self._epilogue(st, l, rows, v)
            return [(lambda: inputs_ready() and resid_ready(all_rows), run1)]
        # stream-K piece: pieces > 0 publish, piece 0 sums all pieces in order
        own = {}

        def run_a():
            for w, u in enumerate(subs):
                rows, v = partial(u)
                if t["ks"] > 0:
                    self._put_slot(("sk", l, t["part_slot"] + t["ks"], w), v)
                else:
                    own[u] = (rows, v)
        phases = [(inputs_ready, run_a)]
        if t["ks"] == 0:
            def ready_b():
                if not all(("sk", l, t["part_slot"] + k, w) in self.slots
                           for k in range(1, t["nks"]) for w in range(len(subs))):
                    return False
                return all(resid_ready(own[u][0]) for u in subs)

            def run_b():
                for w, u in enumerate(subs):
                    rows, v = own[u]
                    v = v.copy()
                    for k in range(1, t["nks"]):
                        v = v + self._take_slot(("sk", l, t["part_slot"] + k, w))
                    self._epilogue(st, l, rows, v)
            phases.append((ready_b, run_b))
        return phases

    def _fin_phases(self, t):
        st, l = t["stage"], t["layer"]
        M = self._stage_rows(st)
        subs = list(range(t["row0"] // 16, t["row0"] // 16 + t["nsub"]))
        ss = self._stage_ss(st, l)

        def ready():
            if not all(("ks", l, t["part_slot"] + u * t["nks"] + k) in self.slots
                       for u in subs for k in range(t["nks"])):
                return False
            if ss and np.isnan(self.buf[ss[0]][ss[1]]).any():
                return False
            if st in (O, DOWN):
                hin = "hres" if st == O else "hmid"
                lo, hi = 16 * subs[0], min(M, 16 * (subs[-1] + 1))
                if not all(self._written(hin, l, n, lo, hi) for n in range(self.b)):
                    return False
            return True

        def run():
            for u in subs:
                rows = [r for r in range(16 * u, 16 * u + 16) if r < M]
                v = None
                for k in range(t["nks"]):
                    p = self._take_slot(("ks", l, t["part_slot"] + u * t["nks"] + k))
                    v = p if v is None else v + p
                self._epilogue(st, l, rows, v)
        return [(ready, run)]

    def _embed_phases(self, t):
        c0, nc = t["row0"], t["nsub"]

        def run():
            E = self._w("model.embed_tokens.weight")
            w0 = self._w("model.layers.0.input_layernorm.weight")
            for n in range(self.b):
                h = E[self.tok[n], c0:c0 + nc]
                self._write("hres", (0, n, slice(c0, c0 + nc)), h)
                self._write("xattn", (0, n, slice(c0, c0 + nc)), h * w0[c0:c0 + nc])
                for j in range(nc // 16):
                    self._write("ssattn", (0, n, c0 // 16 + j), float(np.sum(h[16 * j:16 * j + 16] ** 2)))
        return [(lambda: True, run)]

    # ---- attention partition (as the device cuts it from seq_lens)
    def _partition(self, l, cu):
        b, nkv = self.b, self.nkv
        slen = [p + 1 for p in self.pos]
        W0 = sum(slen) * nkv
        n = (W0 + self.min_rows - 1) // self.min_rows
        nacu = 1 if n < 1 else min(n, self.n_cu)
        cap = self.amap[l][self.n_cu]
        if cap > 0 and nacu > cap and (W0 + cap - 1) // cap <= 256:
            nacu = cap
        pad = min(W0 // (2 * nacu), self.attn_pad)
        if W0 + b * nkv * pad >= (1 << 31):
            pad = 0
        W = W0 + b * nkv * pad
        slot = self.amap[l][cu]
        cu_lo = lambda c: W * c // nacu
        pos = cu_lo(slot) if slot < nacu else W
        hi = cu_lo(slot + 1) if slot < nacu else W
        pieces = []
        while pos < hi:
            acc, i = 0, 0
            for i in range(b):
                seg = nkv * (slen[i] + pad)
                if pos < acc + seg or i == b - 1:
                    break
                acc += seg
            s = slen[i]
            sv = s + pad
            off = pos - acc
            g, jv = off // sv, off % sv
            if jv < pad:
                if hi - pos <= pad - jv:
                    break
                pos += pad - jv
                jv = pad
            take = min(sv - jv, hi - pos)
            j0 = jv - pad
            pieces.append(dict(i=i, g=g, j0=j0, j1=j0 + take, seg_start=acc + g * sv + pad, sid=i * nkv + g))
            pos += take
        cu_of = lambda x: ((x + 1) * nacu + W - 1) // W - 1
        for P in pieces:
            s = slen[P["i"]]
            cf, cl = cu_of(P["seg_start"]), cu_of(P["seg_start"] + s - 1)
            P["npieces"] = cl - cf + 1 if W >= nacu else cu_lo(cl + 1) - cu_lo(cf)
            P["finisher"] = P["npieces"] > 1 and slot == cf
            P["piece_slots"] = [cf + pc if W >= nacu else cu_of(P["seg_start"] + pc) for pc in range(P["npieces"])]
            P["slot"] = slot
        return pieces

    def _qkv_rows(self, l, i, g):
        """q of the group's heads (after QK-norm and RoPE, scaled), k, v of the
        new row, from the step's qkv output."""
        sh, hd, G = self.sh, self.sh.head_dim, self.G
        row = self.buf["qkv"][l, i]
        p = self.pos[i]
        from oracle import rope, rms_norm
        q = row[g * G * hd:(g + 1) * G * hd].reshape(G, hd)
        k = row[self.qdim + g * hd:self.qdim + (g + 1) * hd]
        v = row[self.qdim + self.kvdim + g * hd:self.qdim + self.kvdim + (g + 1) * hd]
        if sh.qk_norm:
            q = rms_norm(q, self._w(f"model.layers.{l}.self_attn.q_norm.weight"), sh.rms_eps)
            k = rms_norm(k, self._w(f"model.layers.{l}.self_attn.k_norm.weight"), sh.rms_eps)
        return rope(q, p, sh.rope_theta) / math.sqrt(hd), rope(k, p, sh.rope_theta), v

    def _attn_phases(self, t, cu):
        l = t["layer"]
        hd, G = self.sh.head_dim, self.G
        holder = {}

        def ready_a():
            pieces = holder.setdefault("p", self._partition(l, cu))
            for P in pieces:
                i, g = P["i"], P["g"]
                if np.isnan(self.buf["qkv"][l, i, g * G * hd:(g + 1) * G * hd]).any():
                    return False
                if P["j1"] == self.pos[i] + 1:  # the new row too
                    if np.isnan(self.buf["qkv"][l, i, self.qdim + g * hd:self.qdim + (g + 1) * hd]).any():
                        return False
                    vo = self.qdim + self.kvdim + g * hd
                    if np.isnan(self.buf["qkv"][l, i, vo:vo + hd]).any():
                        return False
            return True

        def run_a():
            for P in holder["p"]:
                i, g = P["i"], P["g"]
                p = self.pos[i]
                q, k, v = self._qkv_rows(l, i, g)
                Kr = self.K[l, i, g, P["j0"]:min(P["j1"], p)]
                Vr = self.V[l, i, g, P["j0"]:min(P["j1"], p)]
                if P["j1"] == p + 1:
                    self._write("knew", (l, i, g), k)
                    self._write("vnew", (l, i, g), v)
                    Kr = np.concatenate([Kr, k[None]], 0)
                    Vr = np.concatenate([Vr, v[None]], 0)
                z = q @ Kr.T                      # [G, rows]
                m = z.max(-1)
                e = np.exp(z - m[:, None])
                part = (m, e.sum(-1), e @ Vr)
                if P["npieces"] == 1:
                    self._write("aout", (l, i, slice(g * G * hd, (g + 1) * G * hd)),
                                (part[2] / part[1][:, None]).reshape(-1))
                else:
                    self._put_slot(("ap", l, P["slot"] + P["sid"]), part)
        phases = [(ready_a, run_a)]

        def ready_b():
            return all(("ap", l, s + P["sid"]) in self.slots
                       for P in holder["p"] if P["finisher"] for s in P["piece_slots"])

        def run_b():
            for P in holder["p"]:
                if not P["finisher"]:
                    continue
                parts = [self._take_slot(("ap", l, s + P["sid"])) for s in P["piece_slots"]]
                M = np.max([pp[0] for pp in parts], 0)
                lsum = sum(pp[1] * np.exp(pp[0] - M) for pp in parts)
                o = sum(pp[2] * np.exp(pp[0] - M)[:, None] for pp in parts)
                i, g = P["i"], P["g"]
                self._write("aout", (l, i, slice(g * G * hd, (g + 1) * G * hd)), (o / lsum[:, None]).reshape(-1))
        phases.append((ready_b, run_b))
        return phases

    def _program(self, cu):
        ph = []
        for t in self.streams[cu]:
            if t["type"] == T_EMBED:
                ph += self._embed_phases(t)
            elif t["type"] == T_GEMV:
                ph += self._gemv_phases(t)
            elif t["type"] == T_FIN:
                ph += self._fin_phases(t)
            else:
                ph += self._attn_phases(t, cu)
        return ph

    # ------------------------------------------------------------- run
    def run(self, rng):
        pcs = [0] * self.n_cu
        left = sum(len(p) for p in self.prog)
        while left:
            ready = [c for c in range(self.n_cu) if pcs[c] < len(self.prog[c]) and self.prog[c][pcs[c]][0]()]
            if not ready:
                stuck = {c: pcs[c] for c in range(self.n_cu) if pcs[c] < len(self.prog[c])}
                raise Deadlock(f"no CU can proceed: {stuck}")
            c = ready[int(rng.integers(len(ready)))]
            self.prog[c][pcs[c]][1]()
            pcs[c] += 1
            left -= 1
        assert not self.slots, f"partials never consumed: {list(self.slots)[:4]}"
        for k, a in self.buf.items():
            assert not np.isnan(a).any(), f"{k} not fully written"
        self.tokens_out = [int(np.flatnonzero(r == r.max())[0]) for r in self.buf["logits"]]
        return self.buf
