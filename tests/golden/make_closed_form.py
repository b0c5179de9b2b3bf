"""Writes closed_form_cases.json: tiny sampling cases whose expected results
follow by hand from the definitions, computed here with the standard library
only (math, fractions) -- never with the oracle, which these cases pin.

The pages (SonicSampler abstract, English abstract paragraph) name the steps --
penalties, logit bias, grammar mask, temperature, top-k, top-p, min-p -- but
print no worked example, so each case below is built so that every quantity is
exact or a closed form in e:

  * penalty arithmetic on values whose binary32 results are exact (powers of
    two), so the expected processed logits are exact rationals;
  * softmax weights exp(z - zmax) with integer z, so probabilities are ratios
    of powers of e;
  * top-p / min-p cut points chosen far from the thresholds, top-k ties broken
    toward the lower id.

Run:  python tests/golden/make_closed_form.py
"""
import json
import math
import os
from fractions import Fraction

HERE = os.path.dirname(os.path.abspath(__file__))
E = math.e


def norm(ws):
    s = sum(ws)
    return [w / s for w in ws]


def processed_penalties():
    # x = [2, -2, 0.5, 3], history {0, 0, 1}, r = 2, f = 1/4, p = 1/8.
    # id 0 (count 2, x > 0): 2 / 2 = 1;  1 - f*2 = 1/2;  1/2 - 1/8 = 3/8
    # id 1 (count 1, x < 0): -2 * 2 = -4; -4 - 1/4 = -17/4; -17/4 - 1/8 = -35/8
    # ids 2, 3: untouched
    return [float(Fraction(3, 8)), float(Fraction(-35, 8)), 0.5, 3.0]


def processed_bias():
    # x = [0.5, 0, 1], bias entries (2, 1/4), (0, -1/2), (2, 1/2): ids 0 and 2
    # accumulate in array order: id 2: 1 + 1/4 + 1/2 = 7/4; id 0: 1/2 - 1/2 = 0
    return [0.0, 0.0, 1.75]


CASES = [
    {
        "name": "penalties: repetition divides positive and multiplies negative logits once per "
                "distinct id, frequency scales with the count, presence subtracts once",
        "logits": [2.0, -2.0, 0.5, 3.0], "hist": [0, 0, 1], "rep": 2.0, "freq": 0.25, "pres": 0.125,
        "T": 1.0, "top_k": 0, "top_p": 1.0, "min_p": 0.0,
        "processed": processed_penalties(),
        # z = processed; order 3 (3.0), 2 (0.5), 0 (0.375), 1 (-4.375)
        "kept": [3, 2, 0, 1],
        "probs_in_kept_order": norm([1.0, math.exp(0.5 - 3.0), math.exp(0.375 - 3.0),
                                     math.exp(-4.375 - 3.0)]),
    },
    {
        "name": "logit bias: duplicate ids accumulate in array order",
        "logits": [0.5, 0.0, 1.0], "bias_ids": [2, 0, 2], "bias_vals": [0.25, -0.5, 0.5],
        "T": 1.0, "top_k": 0, "top_p": 1.0, "min_p": 0.0,
        "processed": processed_bias(),
        # order: 2 (1.75), then 0 and 1 tie at 0 -> lower id first
        "kept": [2, 0, 1],
        "probs_in_kept_order": norm([1.0, math.exp(-1.75), math.exp(-1.75)]),
    },
    {
        "name": "grammar mask: disallowed tokens become -inf and drop out",
        "logits": [4.0, 1.0, 0.0, 2.0], "mask_allowed": [False, True, True, False],
        "T": 1.0, "top_k": 0, "top_p": 1.0, "min_p": 0.0,
        "processed": [-math.inf, 1.0, 0.0, -math.inf],
        "kept": [1, 2],
        "probs_in_kept_order": norm([1.0, 1.0 / E]),
    },
    {
        "name": "top-p keeps the crossing token: e^2/(e^2+e+1+1/e) = 0.644 < 0.7, adding e gives "
                "0.881 >= 0.7",
        "logits": [2.0, 1.0, 0.0, -1.0], "T": 1.0, "top_k": 0, "top_p": 0.7, "min_p": 0.0,
        "processed": [2.0, 1.0, 0.0, -1.0],
        "kept": [0, 1],
        "probs_in_kept_order": norm([E * E, E]),
    },
    {
        "name": "min-p keeps w = exp(z - zmax) >= 0.3: 1 and 1/e = 0.368 stay, 1/e^2 = 0.135 goes",
        "logits": [0.0, -1.0, -2.0, -3.0], "T": 1.0, "top_k": 0, "top_p": 1.0, "min_p": 0.3,
        "processed": [0.0, -1.0, -2.0, -3.0],
        "kept": [0, 1],
        "probs_in_kept_order": norm([1.0, 1.0 / E]),
    },
    {
        "name": "top-k with ties: the two largest of [1, 3, 3, 0, 3] are ids 1 and 2 (lower ids "
                "first among equal keys)",
        "logits": [1.0, 3.0, 3.0, 0.0, 3.0], "T": 1.0, "top_k": 2, "top_p": 1.0, "min_p": 0.0,
        "processed": [1.0, 3.0, 3.0, 0.0, 3.0],
        "kept": [1, 2],
        "probs_in_kept_order": [0.5, 0.5],
    },
    {
        "name": "temperature: z = x / 0.5 doubles the gaps (exact in binary32); softmax of "
                "[0, -1] / 0.5 is [1, e^-2] normalised",
        "logits": [0.0, -1.0], "T": 0.5, "top_k": 0, "top_p": 1.0, "min_p": 0.0,
        "processed": [0.0, -1.0],
        "kept": [0, 1],
        "probs_in_kept_order": norm([1.0, math.exp(-2.0)]),
    },
    {
        "name": "greedy (T = 0): the lowest id among the maxima",
        "logits": [1.0, 3.0, 3.0, 0.0], "T": 0.0, "top_k": 0, "top_p": 1.0, "min_p": 0.0,
        "processed": [1.0, 3.0, 3.0, 0.0],
        "kept": [1],
        "probs_in_kept_order": [1.0],
    },
    {
        "name": "filters compose in order: top-k 3 of [3, 2, 1, 0], then top-p 0.6 over the "
                "renormalised top-3 (e^3/(e^3+e^2+e) = 0.665 >= 0.6 keeps one token)",
        "logits": [3.0, 2.0, 1.0, 0.0], "T": 1.0, "top_k": 3, "top_p": 0.6, "min_p": 0.0,
        "processed": [3.0, 2.0, 1.0, 0.0],
        "kept": [0],
        "probs_in_kept_order": [1.0],
    },
]


def main():
    out = []
    for c in CASES:
        c = dict(c)
        c["processed"] = [("-inf" if v == -math.inf else v) for v in c["processed"]]
        out.append(c)
    with open(os.path.join(HERE, "closed_form_cases.json"), "w") as f:
        json.dump({"source": "tests/golden/make_closed_form.py (closed forms; no oracle call)",
                   "cases": out}, f, indent=1)


if __name__ == "__main__":
    main()
