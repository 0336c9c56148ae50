"""The CPU oracle against what the pages and the E4M3 format fix
(worked examples, closed forms, invariants, brute force).  CPU only."""
import pytest

import pinlib


@pytest.mark.parametrize("check", pinlib.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(orc, check):
    check(orc)


def test_codec_exhaustive(orc):
    """All 2^32 fp32 bit patterns (NaN/Inf skipped) against the brute-force
    nearest-code search; the round trip covers all 254 finite codes."""
    pinlib.check_codec_exhaustive(orc, stride=1)
