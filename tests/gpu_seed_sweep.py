"""Wide-seed run of the seeded random-shape GPU parity tests (by hand, on a
GPU; not collected by pytest).

    python tests/gpu_seed_sweep.py 1,2,3 [time budget in seconds]

The random-shape tests draw their shapes and data from fixed seeds. This
runs each of them again once per given offset, with every seed the test
draws shifted by 7919 * offset, so the same checks (every output compared
bit for bit with the oracle) cover new shapes. Exits non-zero if any case
fails.
"""
import importlib
import os
import sys
import time
import types

import numpy as _np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import oracle as orc  # noqa: E402

TESTS = [("test_gpu_plan", "test_plan_random_shapes"),
         ("test_gpu_remap", "test_random_shapes"),
         ("test_gpu_dispatch_combine", "test_row_kernels_random_shapes"),
         ("test_gpu_dedup", "test_dedup_random_shapes"),
         ("test_gpu_quant", "test_quant_random_shapes"),
         ("test_gpu_norm", "test_fused_norm_random_shapes"),
         ("test_gpu_chain", "test_zero_copy_random_shapes")]


class _Random:
    """numpy.random with default_rng's seed shifted by the offset."""

    def __init__(self, off):
        self.off = off

    def default_rng(self, seed=None):
        if seed is None:
            return _np.random.default_rng()
        return _np.random.default_rng((int(seed) + 7919 * self.off) % 2 ** 63)

    def __getattr__(self, k):
        return getattr(_np.random, k)


class _Numpy(types.ModuleType):
    def __init__(self, off):
        super().__init__("numpy")
        self.random = _Random(off)

    def __getattr__(self, k):
        return getattr(_np, k)


def main(argv):
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible: the sweep runs the GPU parity tests")
        return 2
    offs = [int(a) for a in argv[0].split(",")] if argv else [1, 2, 3]
    budget = float(argv[1]) if len(argv) > 1 else 600.0
    t0 = time.time()
    fails = runs = 0
    for off in offs:
        for modname, fn in TESTS:
            if time.time() - t0 > budget:
                print("time budget reached", flush=True)
                break
            mod = importlib.import_module(modname)
            real = mod.np
            mod.np = _Numpy(off)
            t1 = time.time()
            runs += 1
            try:
                getattr(mod, fn)(orc)
                print(f"ok   offset={off} {modname}.{fn} {time.time() - t1:.1f}s", flush=True)
            except Exception as ex:  # report every failing test, then go on
                fails += 1
                print(f"FAIL offset={off} {modname}.{fn}: {type(ex).__name__}: {str(ex)[:400]}",
                      flush=True)
            finally:
                mod.np = real
    print(f"{runs - fails} of {runs} test runs passed")
    return 1 if fails else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
