"""CPU oracle for the fused view/reduce path.

TEST INFRASTRUCTURE. This package is a plain, slow, per-node reference
interpreter written from the pages' definitions (see ``interp.py`` for the
passages it follows and the readings it takes). Only the tests, the smoke
check and the benchmark's CPU-baseline leg may import, call, link or run
anything under ``oracle/``; the library's compute path never does, and this
package imports nothing from the library.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, invariants, library routines and brute force on tiny
inputs. No function is left unpinned.
"""

from .interp import (  # noqa: F401
    Interpreter, OracleError, bf16_to_f32, f32_to_bf16, infer, run,
)
