"""The kernels' sigmoid table, as the build writes it, against the oracle (CPU).

The library reads s(g) for bf16 gates from a table of fp32 bit patterns that
swiglu_backward_int8_amd/sigmoid_table.py writes at build time.  This checks,
on the CPU, every entry against the oracle's sigmoid for the same gate, and
that the entries cover every gate whose sigmoid is not saturated (the kernels
clamp the index outside the table); the GPU tests check the kernels' own
lookup over all finite bf16 gates.
"""

import numpy as np

import oracle
from exact import all_finite_bf16
from swiglu_backward_int8_amd import sigmoid_table as st


def _gate_bits(i: int) -> int:
    sign = 1 if i >= st.SIG_L else 0
    return (sign << 15) | (st.SIG_M0 + i - sign * st.SIG_L)


def test_every_entry_equals_the_oracle():
    bits = st.sigma_bits()
    assert len(bits) == 2 * st.SIG_L
    got = np.array(bits, dtype=np.uint32)
    want = np.array([np.float32(oracle.sigmoid(oracle.bf16_to_f32(_gate_bits(i)))) for i in range(len(bits))],
                    dtype=np.float32).view(np.uint32)
    assert np.array_equal(got, want), int((got != want).sum())


def test_clamped_index_covers_every_gate():
    # outside the table's magnitudes the oracle's sigmoid is the clamped entry
    bits = st.sigma_bits()
    for b in all_finite_bf16():
        b = int(b)
        sign, mag = b >> 15, b & 0x7FFF
        k = min(max(mag - st.SIG_M0, 0), st.SIG_L - 1)
        if mag - st.SIG_M0 == k:
            continue  # inside the table: the test above
        want = np.array(np.float32(oracle.sigmoid(oracle.bf16_to_f32(b))), dtype=np.float32).view(np.uint32)
        assert int(want) == bits[sign * st.SIG_L + k], hex(b)


def test_written_initializer(tmp_path):
    path = st.write(str(tmp_path / "sigmoid_table.inc"))
    text = open(path).read()
    words = [int(w.rstrip("u,"), 16) for line in text.splitlines()[1:] for w in line.split()]
    assert words == st.sigma_bits()
