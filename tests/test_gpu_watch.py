"""After the other GPU test files (collected before this one): no wait of
the weight-streaming kernel gave up.  Its hand-over waits are bounded, and
a wait that gives up (a broken invariant) counts itself instead of hanging
the device; the count must be zero after every streaming case above."""
from __future__ import annotations

import pytest

import w8a8_int8_gemm_token_amd as q8

pytestmark = pytest.mark.gpu


def test_stream_waits_never_gave_up():
    assert q8.q8_wait_timeouts() == 0
