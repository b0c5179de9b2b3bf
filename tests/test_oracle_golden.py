"""The oracle against hand-derived closed-form cases (tests/golden/closed_form_cases.json,
written by tests/golden/make_closed_form.py with the standard library only).

Each case fixes its expected processed logits exactly (binary32 arithmetic on
powers of two), its kept set in key order (z descending, lower id first) and its
probabilities as ratios of powers of e. The steps are those the SonicSampler
abstract (English abstract paragraph) lists: penalties, logit bias, grammar
mask, temperature, top-k, top-p, min-p."""
import json
import math
import os

import numpy as np
import pytest

from oracle import pipeline as P

HERE = os.path.dirname(os.path.abspath(__file__))
CASES = json.load(open(os.path.join(HERE, "golden", "closed_form_cases.json")))["cases"]


def pack_allowed(allowed):
    words = np.zeros((len(allowed) + 31) // 32, np.uint32)
    for v, a in enumerate(allowed):
        if a:
            words[v >> 5] |= np.uint32(1 << (v & 31))
    return words


@pytest.mark.parametrize("case", CASES, ids=[c["name"][:40] for c in CASES])
def test_closed_form_case(case):
    x = np.array(case["logits"], np.float32)
    mask = pack_allowed(case["mask_allowed"]) if "mask_allowed" in case else None
    xp = P.process_row(x, np.array(case.get("hist", []), np.int32), case.get("rep", 1.0),
                       case.get("freq", 0.0), case.get("pres", 0.0),
                       np.array(case.get("bias_ids", []), np.int32),
                       np.array(case.get("bias_vals", []), np.float32), mask)
    want = np.array([-np.inf if v == "-inf" else v for v in case["processed"]], np.float32)
    assert np.array_equal(xp.view(np.int32), want.view(np.int32)), (xp, want)
    f = P.filter_row(xp, np.float32(case["T"]), case["top_k"], np.float32(case["top_p"]),
                     np.float32(case["min_p"]))
    assert list(f.kept_ids) == case["kept"]
    got = f.probs[np.array(case["kept"])]
    assert np.allclose(got, case["probs_in_kept_order"], rtol=0, atol=1e-12)
    assert math.isclose(float(f.probs.sum()), 1.0, abs_tol=1e-12)
