"""Loader for the hand-derived worked examples under tests/golden/."""
from __future__ import annotations

import ast
import glob
import json
import math
import os

import numpy as np

from synth import to_bf16_bits

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

_OPS = {ast.Add: lambda a, b: a + b, ast.Sub: lambda a, b: a - b,
        ast.Mult: lambda a, b: a * b, ast.Div: lambda a, b: a / b}


def closed_form(expr: str) -> float:
    """Evaluate a closed-form expression built from numbers, + - * / and exp()."""
    def ev(node):
        if isinstance(node, ast.Expression):
            return ev(node.body)
        if isinstance(node, ast.Constant) and isinstance(node.value, (int, float)):
            return float(node.value)
        if isinstance(node, ast.BinOp) and type(node.op) in _OPS:
            return _OPS[type(node.op)](ev(node.left), ev(node.right))
        if isinstance(node, ast.UnaryOp) and isinstance(node.op, ast.USub):
            return -ev(node.operand)
        if (isinstance(node, ast.Call) and isinstance(node.func, ast.Name)
                and node.func.id == "exp" and len(node.args) == 1):
            return math.exp(ev(node.args[0]))
        raise ValueError(f"unsupported expression: {expr}")
    return ev(ast.parse(str(expr), mode="eval"))


def _tensor(rows, dtype: str) -> np.ndarray:
    """Nested lists of numbers (or "nan") -> float32, or bf16 bits for bf16 cases."""
    a = np.vectorize(float, otypes=[np.float32])(np.array(rows, dtype=object))
    return to_bf16_bits(a) if dtype == "bf16" else a


def cases():
    out = []
    for path in sorted(glob.glob(os.path.join(GOLDEN_DIR, "*.json"))):
        with open(path) as f:
            doc = json.load(f)
        for case in doc["cases"]:
            case = dict(case)
            case["file"] = os.path.basename(path)
            case["cite"] = doc["cite"]
            layers = []
            for lay in case["layers"]:
                layers.append({
                    "role": np.array(lay["role"], dtype=np.uint8),
                    "q": _tensor(lay["q"], case["dtype"]),
                    "k": _tensor(lay["k"], case["dtype"]),
                    "v": _tensor(lay["v"], case["dtype"]),
                    "expect_out": np.array([[[closed_form(e) for e in h] for h in b]
                                            for b in lay["expect_out"]], dtype=np.float64),
                    "expect_S": np.array(lay["expect_S"], dtype=np.int32),
                })
            case["layers"] = layers
            out.append(case)
    return out
