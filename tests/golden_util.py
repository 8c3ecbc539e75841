"""Loader of the hand-worked RoPE + quantisation fixture (tests/golden)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_hand_examples():
    """Rows of rope_quant_hand_examples.txt as tuples
    (name, style, position, weight, {index: value}, e, {index: code}, folded)."""
    rows = []
    with open(os.path.join(GOLDEN, "rope_quant_hand_examples.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            head, xs, e, codes, folded = [p.strip() for p in line.split("|")]
            name, style, pos, w = head.split()
            xs = {int(k): float(v) for k, v in (t.split(":") for t in xs.split())}
            codes = {int(k): int(v, 16) for k, v in (t.split(":") for t in codes.split())}
            rows.append((name, 0 if style == "neox" else 1, int(pos), float(w), xs, int(e),
                         codes, float(folded)))
    return rows
