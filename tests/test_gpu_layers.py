"""Half-layer parity of the bf16 verify pass at full depth, teacher-forced
(tests/helpers_trace.py states the method and the bound).

The verify pass is one forward through every layer ([ZSM] "One pass can score many
tokens"; [LENS] §2.1 step 2).  Cases: the 7B shape at batch 1 (K=5) and batch 8 (K=5)
with per-row cache lengths that differ and end inside 32-key blocks, every layer; the
small model, every layer; the 7B draft shape at the one- and two-row launches of a draft
step, every layer; the 70B shape at layers 0, 40 and 79; 288 rows (batch 32, K=8) at the
first and last layer.  Each case also checks the LM head on the GPU's final rows, and
some report the oracle's own end-to-end logits (not teacher-forced) for comparison.
"""
import pytest
import torch

from speculative_decoding_forward_amd import synth

from helpers_trace import _keep_layers, check_head, check_layers, end_to_end, traced_verify

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ cases ----------

class Test7bBatch1:
    @pytest.fixture(scope="class")
    def t(self):
        wl = synth.WORKLOADS["7b"]
        t = traced_verify(wl.target, 1, wl.K + 1, [wl.ctx], seed=0)
        yield t
        del t
        torch.cuda.empty_cache()

    @pytest.mark.parametrize("half", [0, 1])
    def test_every_layer(self, t, half):
        L = t.shape.n_layers
        check_layers(t, range(half * L // 2, (half + 1) * L // 2))

    def test_head_and_end_to_end(self, t):
        check_head(t)
        end_to_end(t)


class Test7bBatch8Ragged:
    """Per-row cache lengths that differ, several ending inside a 32-key block."""

    @pytest.fixture(scope="class")
    def t(self):
        wl = synth.WORKLOADS["7b"]
        lens = [wl.ctx - 37 * b for b in range(8)]
        t = traced_verify(wl.target, 8, wl.K + 1, lens, seed=1)
        yield t
        del t
        torch.cuda.empty_cache()

    @pytest.mark.parametrize("quarter", [0, 1, 2, 3])
    def test_every_layer(self, t, quarter):
        L = t.shape.n_layers
        check_layers(t, range(quarter * L // 4, (quarter + 1) * L // 4))

    def test_head(self, t):
        check_head(t)


def test_small_every_layer_and_end_to_end():
    wl = synth.WORKLOADS["small"]
    t = traced_verify(wl.target, 1, wl.K + 1, [wl.ctx], seed=2)
    check_layers(t, range(t.shape.n_layers))
    check_head(t)
    end_to_end(t)


@pytest.mark.parametrize("B,M", [(1, 2), (2, 1)])
def test_7b_draft_shape_every_layer(B, M):
    """The draft's forward at the row counts of its steps (two rows when two tokens are
    pending, one row per sequence after that); the draft-step entry point gives bitwise
    these logits (tests/test_gpu_forward.py)."""
    wl = synth.WORKLOADS["7b"]
    t = traced_verify(wl.draft, B, M, [wl.ctx - 5 * b for b in range(B)], seed=3,
                      model_id=synth.DRAFT)
    check_layers(t, range(t.shape.n_layers))
    check_head(t)


def test_70b_layers_0_40_79_and_head():
    wl = synth.WORKLOADS["70b"]
    t = traced_verify(wl.target, 1, wl.K + 1, [wl.ctx], seed=4, keep=_keep_layers([0, 40, 79]))
    check_layers(t, [0, 40, 79])
    check_head(t)
    del t
    torch.cuda.empty_cache()


def test_288_rows_first_and_last_layer():
    """Batch 32 at K=8 (the largest point of the K x batch sweep): five row blocks of up
    to 64 rows on the GEMMs, the normalise pass for every normalised product."""
    wl = synth.WORKLOADS["7b"]
    L = wl.target.n_layers
    lens = [wl.ctx - 3 * b for b in range(32)]
    t = traced_verify(wl.target, 32, 9, lens, seed=5, keep=_keep_layers([0, L - 1]))
    check_layers(t, [0, L - 1])
    check_head(t)
    del t
    torch.cuda.empty_cache()
