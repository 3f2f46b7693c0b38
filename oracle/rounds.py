"""The speculative round as a state machine over a batch of independent rows.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

One round ([CANON] listing "One speculative decoding loop"; [LENS] §2.1 steps 1-3;
[GC] "How It Works" steps 1-4):
  1. the draft proposes x~_0..x~_{K-1} autoregressively, x~_j ~ q_j (uniform purpose 0);
  2. the target scores [y_prev, x~_0..x~_{K-1}] in one call: K+1 rows of logits;
  3. accept / resample / bonus (oracle.sampling.accept_resample_logits);
  4. caches are rolled back to the committed tokens.

Cache invariant (our reading; the pages do not discuss caches beyond [LENS] §3.4): with
n tokens committed for a row, the target cache holds the first n-1 and the last one
(y_prev) is fed at the start of the next verify.  The draft cache holds n-1 or n-2 of
them; the rest are its "pending" tokens, consumed by the first draft step of the round.
After a round that accepted a drafts:
  a < K:  len_t = n-1 + a+1, len_d = len_t, draft pending = [y]
  a = K:  len_t = n-1 + K+1, len_d = len_t - 1, draft pending = [x~_{K-1}, y]
A row whose status is non-zero (nothing emitted) keeps its lengths and pending tokens.
"""
import numpy as np

from . import philox
from .model import KVCache, forward
from .sampling import accept_resample_logits, draft_sample


class SpecRows:
    def __init__(self, tcfg, Wt, dcfg, Wd, ctx, K, max_len, temperature=1.0, top_k=0,
                 top_p=1.0, seed=0):
        ctx = np.asarray(ctx, dtype=np.int64)
        self.B, n0 = ctx.shape
        assert n0 >= 1
        self.tcfg, self.Wt, self.dcfg, self.Wd = tcfg, Wt, dcfg, Wd
        self.K = int(K)
        self.knobs = dict(temperature=temperature, top_k=top_k, top_p=top_p)
        self.seed = int(seed)
        self.round = 0
        self.tcache = KVCache(tcfg, self.B, max_len)
        self.dcache = KVCache(dcfg, self.B, max_len)
        if n0 > 1:
            forward(tcfg, Wt, self.tcache, ctx[:, :-1])
            forward(dcfg, Wd, self.dcache, ctx[:, :-1])
        self.y_prev = ctx[:, -1].copy()
        self.pending = [[int(ctx[b, -1])] for b in range(self.B)]
        self.tokens = [list(map(int, ctx[b])) for b in range(self.B)]
        self.history = []

    def draft(self):
        """K draft steps; returns (x~ [B, K], draft logits [B, K, V])."""
        B, K = self.B, self.K
        V = int(self.dcfg["vocab"] if isinstance(self.dcfg, dict) else self.dcfg.vocab)
        xt = np.zeros((B, K), dtype=np.int64)
        qlog = np.zeros((B, K, V))
        for j in range(K):
            if j == 0:
                n_tok = np.array([len(p) for p in self.pending])
                toks = np.zeros((B, 2), dtype=np.int64)
                for b, p in enumerate(self.pending):
                    toks[b, :len(p)] = p
            else:
                n_tok = np.ones(B, dtype=np.int64)
                toks = xt[:, j - 1:j]
            lg = forward(self.dcfg, self.Wd, self.dcache, toks, n_tok)
            for b in range(B):
                row = lg[b, n_tok[b] - 1].astype(np.float32)
                qlog[b, j] = row
                u = philox.uniform(self.seed, self.round, j, b, philox.PURPOSE_DRAFT)
                xt[b, j] = draft_sample(row, float(u), **self.knobs)
        return xt, qlog

    def verify(self, xt):
        """One target call over [y_prev, x~_0..x~_{K-1}]; returns logits [B, K+1, V]."""
        vt = np.concatenate([self.y_prev[:, None], xt], axis=1)
        return forward(self.tcfg, self.Wt, self.tcache, vt)

    def accept(self, plog, qlog, xt, len_t0, len_d0):
        """Rule + cache roll-back for every row; returns (tokens per row, n_out, a, status)."""
        B, K = self.B, self.K
        j = np.arange(K)
        out = []
        n_out = np.zeros(B, dtype=np.int64)
        acc = np.zeros(B, dtype=np.int64)
        status = np.zeros(B, dtype=np.int64)
        new_t = self.tcache.len.copy()
        new_d = self.dcache.len.copy()
        for b in range(B):
            u_acc = philox.uniform(self.seed, self.round, j, b, philox.PURPOSE_ACCEPT)
            u_res = philox.uniform(self.seed, self.round, np.arange(K + 1), b,
                                   philox.PURPOSE_RESAMPLE)
            toks, n, a, st = accept_resample_logits(
                plog[b].astype(np.float32), qlog[b], xt[b], u_acc, u_res, **self.knobs)
            out.append(toks)
            n_out[b], acc[b], status[b] = n, a, st
            if n == 0:
                new_t[b], new_d[b] = len_t0[b], len_d0[b]
                continue
            new_t[b] = len_t0[b] + a + 1
            if a < K:
                new_d[b] = new_t[b]
                self.pending[b] = [toks[-1]]
            else:
                new_d[b] = new_t[b] - 1
                self.pending[b] = [int(xt[b, K - 1]), toks[-1]]
            self.y_prev[b] = toks[-1]
            self.tokens[b].extend(toks)
        self.tcache.rollback(new_t)
        self.dcache.rollback(new_d)
        return out, n_out, acc, status

    def step(self):
        len_t0 = self.tcache.len.copy()
        len_d0 = self.dcache.len.copy()
        xt, qlog = self.draft()
        plog = self.verify(xt)
        res = self.accept(plog, qlog, xt, len_t0, len_d0)
        self.history.append(dict(xt=xt, qlog=qlog, plog=plog, out=res[0], n_out=res[1],
                                 a=res[2], status=res[3]))
        self.round += 1
        return res
