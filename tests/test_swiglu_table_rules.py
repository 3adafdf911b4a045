"""The SwiGLU-fused tiled preparation looks silu up instead of evaluating it per gate: it
tabulates silu over the bf16 gates with exponent field 103..133 and uses a rule on every
other finite gate -- g/2 below that range (e^-g rounds to 1, the divisor to 2), g above it
for g > 0 and -0 above it for g < 0.  The table itself is filled by the same silu the
direct path evaluates.  This checks each rule against the oracle's silu (reading R14) on
every finite bf16 pattern it covers, and that the window and the rules partition the
finite patterns."""
import numpy as np

import oracle

ELO, SPAN = 103, 31  # exponent fields 103..133, both signs


def _f32_bits(v):
    return int(np.array(v, dtype=np.float32).view(np.uint32))


def test_silu_rules_outside_the_table_window_match_the_oracle():
    ruled = tabled = 0
    for b in range(1 << 16):
        e = (b >> 7) & 0xFF
        if e == 0xFF:
            continue  # infinities and NaN take the direct evaluation
        sign = b >> 15
        g = np.array(b << 16, dtype=np.uint32).view(np.float32)
        if ELO <= e < ELO + SPAN:
            tabled += 1
            continue
        s = _f32_bits(oracle.silu(float(g)))
        if e < ELO:
            want = _f32_bits(np.float32(g) * np.float32(0.5))
        else:
            want = 0x80000000 if sign else _f32_bits(g)
        assert s == want, f"bf16 0x{b:04x}: oracle silu 0x{s:08x}, rule 0x{want:08x}"
        ruled += 1
    assert tabled == 2 * SPAN * 128
    assert ruled + tabled == 2 * 255 * 128


def test_silu_window_needs_the_table_at_both_ends():
    """The window is no wider than it must be at its ends: at exponent 103 and 133 some
    gates of one sign already break the rule the other side would apply."""
    def breaks(e, sign, rule):
        for m in range(128):
            b = (sign << 15) | (e << 7) | m
            g = np.array(b << 16, dtype=np.uint32).view(np.float32)
            s = _f32_bits(oracle.silu(float(g)))
            want = _f32_bits(np.float32(g) * np.float32(0.5)) if rule == "half" else (
                0x80000000 if sign else _f32_bits(g))
            if s != want:
                return True
        return False
    assert breaks(ELO, 0, "half")             # the positive gates at 103 need the table
    assert breaks(ELO + SPAN - 1, 1, "large")  # and so do the negative ones at 133
