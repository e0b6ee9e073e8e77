"""The layer-by-layer composition of the oracle's ops (toy_layer_oracle.py)
against the oracle's own toy forward: the same ops in the same order, so the
logits must agree bit for bit.  This is what lets the GPU test hold each of the
driver's layers, fed the GPU's own input bits, to the per-op bar."""
from __future__ import annotations

import numpy as np
import pytest

import toy_layer_oracle as TL
from invariant_bi_rmsnorm_amd import inputs as I

SMALL = dict(layers=3, hidden=128, heads=4, kv_heads=2, head_dim=32, mlp=192, vocab=97,
             eps=1e-6, rope_theta=10000.0)


@pytest.mark.parametrize("T", [1, 5, 23])
def test_layer_composition_equals_oracle_toy_forward(orc, T):
    w = I.toy_weights(SMALL, seed=3)
    ids = I.rng(77, T).integers(0, SMALL["vocab"], size=T).astype(np.int32)
    ref = orc.toy_forward(SMALL, w, ids)
    got = TL.forward(orc, SMALL, w, ids)
    assert np.array_equal(got.view(np.uint64), ref.view(np.uint64))


def test_layer_composition_sees_a_wiring_change(orc):
    """A plausible wiring slip (gate and up halves swapped) changes the logits:
    the exact-equality pin above would catch it in either implementation."""
    w = I.toy_weights(SMALL, seed=3)
    ids = I.rng(78).integers(0, SMALL["vocab"], size=9).astype(np.int32)
    ref = orc.toy_forward(SMALL, w, ids)
    F = SMALL["mlp"]
    w2 = dict(w, layers=[dict(lw, wgu=np.concatenate([lw["wgu"][F:], lw["wgu"][:F]])) for lw in w["layers"]])
    assert not np.array_equal(TL.forward(orc, SMALL, w2, ids), ref)
