"""Load the hand-worked fixtures under tests/golden and evaluate their closed forms."""
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
_NS = {"exp": math.exp, "log": math.log, "inf": math.inf, "__builtins__": {}}


def closed_form(expr: str) -> float:
    return float(eval(expr, _NS))  # expressions are fixed strings from the fixture files


def evaluate(tree):
    if isinstance(tree, list):
        return [evaluate(x) for x in tree]
    return closed_form(tree)


def load(name: str) -> list:
    with open(os.path.join(GOLDEN, name)) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        c["out_expected"] = np.array(evaluate(c["out"]), dtype=np.float64)
        c["lse_expected"] = np.array(evaluate(c["lse"]), dtype=np.float64)
    return cases
