"""Run every oracle pin against another build of oracle.c; print the failing pins as JSON.

Used by test_oracle_mutants.py in a child process (a planted mistake may crash).
Usage: python tests/mutant_runner.py /path/to/liboracle_mutant.so
"""
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402

oracle.use_library(sys.argv[1])
import test_oracle_pins as pins  # noqa: E402

failed = []
for name in sorted(dir(pins)):
    if not name.startswith("test_"):
        continue
    fn = getattr(pins, name)
    cases = [()]
    if name == "test_bf16_round_known_values":
        cases = pins.GOLD_BF16
    for args in cases:
        try:
            fn(oracle, *args)
        except Exception as e:  # noqa: BLE001 - any failure counts as detection
            failed.append(f"{name}{list(args) if args else ''}: {type(e).__name__}")
            break
print(json.dumps(failed))
