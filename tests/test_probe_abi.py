"""Host-side checks of the MFMA probe's C ABI (no GPU): every argument check
returns its status before any launch."""
import pytest

import headwise_chunked_context_amd as hc_amd
from headwise_chunked_context_amd import binding as B

P = 0x7F0000000000
MIB16 = 16 << 20


@pytest.mark.parametrize("args", [
    (None, MIB16, 10, 512, P, P),
    (P, MIB16, 10, 512, None, P),
    (P, MIB16, 10, 512, P, None),
    (P, MIB16 - 2, 10, 512, P, P),        # less than 16 MiB of operands
    (P, MIB16, 0, 512, P, P),             # no rounds
    (P, MIB16, 10, 0, P, P),              # no workgroups
    (P, MIB16, 10, (1 << 22) + 1, P, P),  # too many workgroups
    (P + 8, MIB16, 10, 512, P, P),        # operands not 16-byte aligned
    (P, MIB16, 10, 512, P + 2, P),        # sink not 4-byte aligned
    (P, MIB16, 10, 512, P, P + 4),        # clocks not 8-byte aligned
])
def test_probe_checks_before_any_launch(args):
    assert hc_amd.lib().upipe_probe_mfma(*args, None) == B.UPIPE_EINVAL


def test_probe_flop_count():
    # 32 MFMAs of 32 x 32 x 16 per wave and round, 2 FLOP per multiply-add
    assert B.PROBE_FLOP_PER_ROUND == 32 * 32768
