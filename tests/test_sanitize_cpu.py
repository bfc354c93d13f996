"""The host code of the C ABI (validation, workspace carving, launch set-up)
under AddressSanitizer and UndefinedBehaviorSanitizer: the build module's
--sanitize mode compiles an instrumented copy of the library (device code
unchanged) and runs tests/test_abi_cpu.py against it.  No GPU is used."""
import shutil

import pytest

from latent_flow_matching_flux_amd import build


@pytest.mark.slow
@pytest.mark.skipif(shutil.which(build.HIPCC) is None, reason="hipcc not installed")
def test_abi_host_code_clean_under_sanitizers():
    assert build.sanitize_check() == 0
