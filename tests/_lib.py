"""Load the built HIP library for the tests, building it first only if it is missing."""
import os

from speculative_decoding_05_amd import build as _build

if not os.path.exists(_build.LIB):
    _build.build()

from speculative_decoding_05_amd import binding as mb  # noqa: E402,F401
