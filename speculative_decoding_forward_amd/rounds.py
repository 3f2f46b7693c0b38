"""Speculative rounds on one GPU: the sequence of C-ABI calls that makes one round.

One round ([CANON] listing "One speculative decoding loop"; [LENS] §2.1 steps 1-3;
[GC] "How It Works" steps 1-4):
  1. K draft steps (spec_draft_step): x~_j ~ q_j;
  2. verify-input assembly (spec_verify_tokens) and ONE target call over
     [y_prev, x~_0..x~_{K-1}] (spec_verify_forward);
  3. accept / resample / bonus with in-place cache roll-back and the next round's
     pending tokens (spec_accept_resample).
Every step runs in the HIP library; this class only owns the device buffers and issues
the calls on one stream.  All state stays on the device between rounds, including the
round number (an int64 device counter advanced by the accept step), so one round can be
captured as a HIP graph and replayed round after round (``capture`` / ``replay``).
"""
import numpy as np
import torch

from . import binding

PREFILL_CHUNK = 64


class SpecDecoder:
    def __init__(self, tshape, tweights, dshape, dweights, batch, K, max_len, knobs, seed=0,
                 device="cuda", prefill_chunk=PREFILL_CHUNK, models=None, caches=None):
        """models = (target, draft) binding.Model and caches = (target, draft)
        binding.KVCache already built (the weights arguments are then unused): several
        decoders -- e.g. one per K -- can share one copy of the models and one prefilled
        context."""
        if tshape.vocab != dshape.vocab:
            raise ValueError("draft and target must share the vocabulary")
        self.B, self.K, self.max_len = batch, K, max_len
        self.knobs, self.seed, self.device = tuple(knobs), int(seed), device
        self.chunk = prefill_chunk
        V = tshape.vocab
        if models is not None:
            self.target, self.draft = models
        else:
            self.target = binding.Model(tshape, tweights)
            self.draft = binding.Model(dshape, dweights)
        if caches is not None:
            self.tkv, self.dkv = caches
            if self.tkv.max_len < max_len or self.dkv.max_len < max_len:
                raise ValueError("shared caches are shorter than max_len")
        else:
            self.tkv = binding.KVCache(tshape, batch, max_len, device)
            self.dkv = binding.KVCache(dshape, batch, max_len, device)
        rows = max(K + 1, prefill_chunk)
        self.ws_t = self.target.workspace(batch, rows, max_len, device)
        self.ws_d = self.draft.workspace(batch, rows, max_len, device)
        i32 = dict(dtype=torch.int32, device=device)
        self.x_tilde = torch.zeros((batch, K), **i32)
        self.q_logits = torch.zeros((batch, K, V), dtype=torch.float32, device=device)
        self.p_logits = torch.zeros((batch, K + 1, V), dtype=torch.float32, device=device)
        self.vtok = torch.zeros((batch, K + 1), **i32)
        self.out_tok = torch.zeros((batch, K + 1), **i32)
        self.n_out = torch.zeros(batch, **i32)
        self.row_status = torch.zeros(batch, **i32)
        self.pending = torch.zeros((batch, 2), **i32)
        self.n_pending = torch.ones(batch, **i32)
        self.acc_ws = binding.accept_workspace(batch, K, device)
        self.round_dev = torch.zeros(1, dtype=torch.int64, device=device)
        self.graph = None
        self.prefill_logits = torch.zeros((batch, prefill_chunk, V), dtype=torch.float32,
                                          device=device)

    def prefill(self, ctx, stream=None):
        """Commit the context ids ctx [B, n] (n >= 1): the first n-1 go into both caches
        in chunks, the last becomes the pending token of both models."""
        ctx = np.asarray(ctx, dtype=np.int32)
        B, n = ctx.shape
        assert B == self.B and n >= 1
        for s in range(0, n - 1, self.chunk):
            e = min(n - 1, s + self.chunk)
            tok = torch.from_numpy(np.ascontiguousarray(ctx[:, s:e])).to(self.device)
            lg = self.prefill_logits[:, : e - s].contiguous() if e - s < self.chunk \
                else self.prefill_logits
            binding.verify_forward(self.target, self.tkv, tok, lg, self.ws_t, stream=stream)
            binding.verify_forward(self.draft, self.dkv, tok, lg, self.ws_d, stream=stream)
        self.pending[:, 0] = torch.from_numpy(ctx[:, -1].copy()).to(self.device)
        self.pending[:, 1] = -1
        self.n_pending.fill_(1)

    def draft_phase(self, rnd, stream=None, device_round=False):
        rd = self.round_dev if device_round else None
        for j in range(self.K):
            binding.draft_step(self.draft, self.dkv, self.pending, self.n_pending, j, self.knobs,
                               self.seed, rnd, self.x_tilde, self.q_logits, self.ws_d,
                               stream=stream, round_dev=rd)

    def verify_phase(self, stream=None):
        binding.verify_tokens(self.pending, self.n_pending, self.x_tilde, self.vtok,
                              stream=stream)
        binding.verify_forward(self.target, self.tkv, self.vtok, self.p_logits, self.ws_t,
                               stream=stream)

    def accept_phase(self, rnd, stream=None, device_round=False):
        binding.accept_resample(self.p_logits, self.q_logits, self.x_tilde, self.knobs,
                                self.seed, rnd, self.out_tok, self.n_out, self.row_status,
                                self.acc_ws, tkv=self.tkv, dkv=self.dkv, pending=self.pending,
                                n_pending=self.n_pending, stream=stream,
                                round_dev=self.round_dev if device_round else None)

    def step(self, rnd, stream=None):
        """One full round with round number `rnd` (asynchronous on the stream)."""
        self.draft_phase(rnd, stream)
        self.verify_phase(stream)
        self.accept_phase(rnd, stream)

    def step_device_round(self, stream=None):
        """One full round numbered by the device counter, which it then advances."""
        self.draft_phase(0, stream, device_round=True)
        self.verify_phase(stream)
        self.accept_phase(0, stream, device_round=True)

    def set_round(self, rnd):
        self.round_dev.fill_(int(rnd))

    def capture(self):
        """Capture one device-numbered round as a HIP graph (nothing is executed)."""
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step_device_round()
        self.graph = g
        return g

    def replay(self):
        """Run the captured round once more (the device round counter numbers it)."""
        self.graph.replay()
