"""Reader for the small text fixtures under tests/golden/ ("key: values")."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = line.split(":", 1)
            vals = val.split()
            try:
                nums = [int(v) for v in vals]
            except ValueError:
                nums = [float(v) for v in vals]
            out[key.strip()] = nums[0] if len(nums) == 1 else nums
    return out
