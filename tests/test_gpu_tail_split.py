"""The down projection's last-round split against the CPU oracle.

When the down projection's tiles fill at least one round of resident
workgroups and leave a last round at most half full, the tiles of that
round are cut along k into pieces; the later pieces' partial tiles are added
to the first piece's in a fixed order by a second kernel, which writes the
fp32 partials (several chosen groups) or Y (one).  Here the round
size is set small (CEFN_TAIL_SLOTS) so that layers of test size take that
path, with the split count the plan picks checked on the host first.

Bars: outputs within 1e-2 of max|y_ref| (16-bit layers), two calls bit for
bit identical, and within the same bar of the same layer without the split.
"""
import math

import numpy as np
import pytest

from compressed_expert_ffn_amd.workloads import WORKLOADS
from oracle import moe_oracle as O
from tests.gpu_util import TOL, rel_err, say, x_to_device, y_to_host
from tests.layers import make_parity_layer
from tests.test_gpu_combos import combo_workload

pytestmark = pytest.mark.gpu


def plan(total: int, slots: int, smax: int, KT: int):
    """(whole tiles, tail tiles, pieces per tail tile) as the kernels plan
    them (no room limit: the tests' layers have room for every piece)."""
    if slots <= 0 or total <= slots:
        return total, 0, 1
    tail = total % slots
    if tail == 0 or 2 * tail > slots:
        return total, 0, 1
    S = min(smax, slots // tail, KT // 4)
    if S < 2:
        return total, 0, 1
    return total - tail, tail, S


def slots_for(total: int, KT: int):
    """The round size under which `total` tiles leave the most pieces in a
    split last round."""
    best = None
    for s in range(4, total):
        F, tail, S = plan(total, s, 8, KT)
        if tail and S >= 2 and F >= s and (best is None or tail * S >= best[1] * best[2]):
            best = (s, tail, S)
    assert best is not None, f"no round size splits {total} tiles"
    return best


def _workload(case):
    kind, T, bm = case
    if kind == "combo":
        # 16-bit residual tail in the first piece, two groups per token
        return combo_workload("swiglu", "bf16", "f16", "f16", 16, (4, 4), 2, 2, T, d=256, f=1024), bm
    return WORKLOADS[kind].with_T(T), bm


# two chosen groups (fp32 partials and the combine after the fixup) and one
# chosen group (the fixup writes Y), 16-bit and INT4 residual tails included
CASES = [(2, 300, 128), (2, 520, 256), (4, 64, 32), ("combo", 257, 64), (1, 700, 128), (3, 1000, 128),
         (3, 600, 64)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-T{c[1]}-bm{c[2]}" for c in CASES])
def test_last_round_split_matches_oracle(case, monkeypatch):
    from compressed_expert_ffn_amd import _lib as L
    w, bm = _workload(case)
    wT, inputs, layer = make_parity_layer(w)
    rt = O.route(layer)
    gcounts = O.permutation(rt["gidx"], wT.G)[0]
    total = int(sum(math.ceil(int(c) / bm) for c in gcounts)) * math.ceil(wT.d / 256)
    slots, tail, S = slots_for(total, wT.f // 64)
    say(f"[tail split] {wT.name} T={wT.T} bm={bm}: {total} tiles, round {slots}, "
        f"{tail} tail tiles in {S} pieces")
    for k, v in {"CEFN_BM_G2": str(bm), "CEFN_KS_G2": "1", "CEFN_G2K": "0"}.items():
        monkeypatch.setenv(k, v)
    X = x_to_device(inputs["X"], w.x_dtype)
    toks = np.sort(np.random.default_rng(11).choice(wT.T, size=min(wT.T, 40), replace=False))
    ref = O.forward(layer, tokens=toks)
    outs = {}
    for name, s in (("split", slots), ("whole", 0)):
        monkeypatch.setenv("CEFN_TAIL_SLOTS", str(s))
        lay = L.Layer(L.config_from_workload(wT), inputs)
        try:
            y1 = y_to_host(lay.forward(X))
            y2 = y_to_host(lay.forward(X))
        finally:
            lay.close()
        assert np.array_equal(y1.view(np.uint64), y2.view(np.uint64)), f"{name}: repeat calls differ"
        err = rel_err(y1[toks], ref)
        say(f"[tail split] {name}: rel err {err:.3e}")
        assert err <= TOL[w.x_dtype]
        outs[name] = y1
    assert rel_err(outs["split"], outs["whole"]) <= TOL[w.x_dtype]
