"""Reader for tests/golden/hand_cases.json (plain JSON, no code executed)."""

import json
import math
import pathlib

import numpy as np

GOLDEN = pathlib.Path(__file__).resolve().parent / "golden" / "hand_cases.json"
BITS = {"float32": np.uint32, "float16": np.uint16, "bfloat16": np.uint16}


def load():
    return json.loads(GOLDEN.read_text())


def parse_value(s: str) -> float:
    if s.startswith(("0x", "-0x")):
        return float.fromhex(s)
    return float(s)


def parse_ranges(spec: str):
    out = set()
    for part in filter(None, spec.split(",")):
        if "-" in part:
            a, b = part.split("-")
            out.update(range(int(a), int(b) + 1))
        else:
            out.add(int(part))
    return out


def build_case(case, seed=0):
    """(logits bits, mask int32) arrays for one golden case; logits random."""
    rng = np.random.default_rng(seed)
    dt = BITS[case["dtype"]]
    hi = 2**32 if dt == np.uint32 else 2**16
    logits = rng.integers(0, hi, size=(case["rows"], case["cols"]), dtype=np.uint64).astype(dt)
    rows = []
    for r in case["mask"]:
        if isinstance(r, dict):
            words = [int(r["default"], 16)] * case["mask_cols"]
            for k, v in r["set"].items():
                words[int(k)] = int(v, 16)
        else:
            words = [int(w, 16) for w in r]
        assert len(words) == case["mask_cols"]
        rows.append(words)
    mask = np.array(rows, dtype=np.uint64).astype(np.uint32).view(np.int32)
    return logits, mask


def expected_positions(case):
    return {int(r): parse_ranges(spec) for r, spec in case["masked"].items()}


def fill_of(case):
    return parse_value(case["fill"]) if case["fill"] not in ("-inf", "inf") else (
        -math.inf if case["fill"] == "-inf" else math.inf)
