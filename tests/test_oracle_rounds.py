"""Pins of the oracle's round state machine (draft K, verify, accept, roll back)."""
import numpy as np
import pytest

from oracle import model, rounds
from speculative_decoding_forward_amd import synth


def tiny():
    return synth.WORKLOADS["tiny"]


@pytest.fixture(scope="module")
def tiny_weights():
    wl = tiny()
    Wt = synth.weights_to_numpy(synth.make_weights(wl.target, seed=0, model_id=synth.TARGET))
    Wd = synth.weights_to_numpy(synth.make_weights(wl.draft, seed=0, model_id=synth.DRAFT))
    return Wt, Wd


def test_draft_equal_to_target_accepts_everything(tiny_weights):
    """With the target as its own draft, q = p at every position, so every draft is
    accepted and each call emits K+1 tokens; any slip in the cache or pending-token
    bookkeeping would make q differ from p and show up as a rejection."""
    wl = tiny()
    Wt, _ = tiny_weights
    ctx = synth.context_ids(0, 2, wl.ctx, wl.target.vocab)
    st = rounds.SpecRows(wl.target, Wt, wl.target, Wt, ctx, wl.K, max_len=128, seed=0)
    for r in range(6):
        toks, n_out, a, status = st.step()
        assert np.all(n_out == wl.K + 1) and np.all(status == 0)
    assert np.array_equal(st.tcache.len, wl.ctx - 1 + 6 * (wl.K + 1) * np.ones(2))
    assert np.array_equal(st.dcache.len, st.tcache.len - 1)


def test_tiny_rounds_invariants_and_cache_consistency(tiny_weights):
    """The tiny workload (fp32 2-layer target, 1-layer draft, K=4, T=1): bounds on n_out,
    cache lengths, and the target cache after each round equal to a fresh prefill of
    the committed tokens."""
    wl = tiny()
    Wt, Wd = tiny_weights
    ctx = synth.context_ids(0, 1, wl.ctx, wl.target.vocab)
    st = rounds.SpecRows(wl.target, Wt, wl.draft, Wd, ctx, wl.K, max_len=256, seed=0)
    total = 0
    for r in range(8):
        toks, n_out, a, status = st.step()
        assert 1 <= n_out[0] <= wl.K + 1 and status[0] == 0
        total += int(n_out[0])
        committed = np.array(st.tokens[0])
        assert committed.size == wl.ctx + total
        assert st.tcache.len[0] == committed.size - 1
        assert st.dcache.len[0] + len(st.pending[0]) == committed.size
        # next-token logits from the rolled-back cache equal a fresh recompute
        c = st.tcache.copy()
        nxt = model.forward(wl.target, Wt, c, committed[None, -1:])
        fresh = model.forward(wl.target, Wt, model.KVCache(wl.target, 1, 256),
                              committed[None])
        np.testing.assert_allclose(nxt[0, 0], fresh[0, -1], rtol=0, atol=1e-10)
        cd = st.dcache.copy()
        pend = np.array(st.pending[0])[None]
        dn = model.forward(wl.draft, Wd, cd, pend)
        dfresh = model.forward(wl.draft, Wd, model.KVCache(wl.draft, 1, 256), committed[None])
        np.testing.assert_allclose(dn[0, -1], dfresh[0, -1], rtol=0, atol=1e-10)


@pytest.mark.parametrize("draft_is_target", [False, True])
def test_greedy_rounds_emit_the_targets_own_argmax_decoding(tiny_weights, draft_is_target):
    """At T = 0 the method changes no output: whatever the draft proposes, the committed
    tokens equal the target's own one-token-at-a-time argmax decoding (the argmax column
    of the speedup table in [LENS] "How much faster in practice?" compares against exactly
    that).  A slip in the accept test, the resample or the cache roll-back changes the
    sequence."""
    wl = tiny()
    Wt, Wd = tiny_weights
    B, n_rounds = 2, 6
    ctx = synth.context_ids(3, B, wl.ctx, wl.target.vocab)
    dshape, dW = (wl.target, Wt) if draft_is_target else (wl.draft, Wd)
    st = rounds.SpecRows(wl.target, Wt, dshape, dW, ctx, wl.K, max_len=256,
                         temperature=0.0, seed=0)
    for _ in range(n_rounds):
        toks, n_out, a, status = st.step()
        assert np.all(status == 0)
        if draft_is_target:
            assert np.all(n_out == wl.K + 1)
    for b in range(B):
        new = st.tokens[b][wl.ctx:]
        cache = model.KVCache(wl.target, 1, 256)
        lg = model.forward(wl.target, Wt, cache, ctx[b:b + 1])
        ref = []
        while len(ref) < len(new):
            ref.append(int(np.argmax(lg[0, -1].astype(np.float32))))
            lg = model.forward(wl.target, Wt, cache, np.array([[ref[-1]]]))
        assert new == ref
