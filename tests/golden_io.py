"""Reader for the text fixtures under tests/golden/ (``key = values`` lines, ``#`` comments)."""

import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, _, val = line.partition("=")
            parts = val.split()
            nums = []
            for p in parts:
                try:
                    nums.append(int(p))
                except ValueError:
                    nums.append(float(p))
            out[key.strip()] = nums if len(nums) != 1 else nums[0]
    return out
