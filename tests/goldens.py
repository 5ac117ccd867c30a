"""Reader of the small text fixtures under tests/golden/ (sections of key = values)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    cases, cur = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("[") and line.endswith("]"):
                cur = cases.setdefault(line[1:-1], {})
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            cur[key] = val.split()
    return cases
