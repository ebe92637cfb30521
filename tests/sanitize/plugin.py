"""pytest plugin for the sanitizer run (tests/test_sanitizers.py): points the oracle
wrapper and the libsscan binding at the AddressSanitizer/UBSan builds named in the
environment, before any test loads a library."""
import os

import oracle
from state_space_model_sscan_amd import binding

oracle._LIB = os.environ["SSCAN_SAN_ORACLE"]
binding.LIB_PATH = os.environ["SSCAN_SAN_LIBSSCAN"]
