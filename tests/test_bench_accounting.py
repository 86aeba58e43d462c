"""The bench's algorithmic accounting (host logic, no GPU).

The bytes a call must move at least once, per workload: u, Delta (and z)
read and y written once per (b, l, d), B and C once per (b, l, n), A, D and
bias once, h_last once where returned; the decode step reads and writes the
fp32 state once.  The figures are the workload table's (batch 1/8/1/16,
L 256/2048/131072/2048, D 64/1536/2048/5120, N 16; the decode step batch
256, D 5120), computed here by hand from those shapes.
"""
import bench


def test_forward_algorithmic_bytes():
    # tiny: fp32, no gate: 16384 elems x (u, Delta, y) 12 B + B, C + A + D, bias
    assert bench.algorithmic_bytes(1, 256, 64, 16, 4, False) == \
        16384 * 12 + 2 * 256 * 16 * 4 + 64 * 16 * 4 + 2 * 64 * 4 == 233_984
    assert bench.algorithmic_bytes(8, 2048, 1536, 16, 2, True) == 202_485_760
    assert bench.algorithmic_bytes(1, 131072, 2048, 16, 2, True, with_last=True) == \
        2_156_150_784
    assert bench.algorithmic_bytes(16, 2048, 5120, 16, 2, True) == 1_344_643_072


def test_decode_bytes_per_step():
    # state read + written (167.8 MB) and the per-token inputs and output
    assert bench.decode_bytes(256, 5120, 16, 2, True) == 178_642_944


def test_valu_slot_counts():
    # forward: 4 N per state plus the per-element work (bf16, gated)
    assert bench.algorithmic_valu_slots(16, True, 2) == 87
    assert bench.algorithmic_valu_slots(16, True, 2) - bench.algorithmic_valu_slots(8, True, 2) \
        == 4 * 8
    # general A: an exp2 (3 slots) per state for the power chain's multiply,
    # and no exp of Delta A[d,0]: 6 N + 20
    assert bench.algorithmic_valu_slots(16, True, 2, general_a=True) == 116
    # forward variants: reverse is addressing only; exact ZOH 3 N + 8 more
    # (the running power sum, its product with B, the scale; the coefficient
    # em per element), the conv prologue k taps and SiLU (k + 6)
    assert bench.algorithmic_valu_slots(16, True, 2, flags=2) == 87
    assert bench.algorithmic_valu_slots(16, True, 2, flags=1) == 87 + 48 + 8
    assert bench.algorithmic_valu_slots(16, True, 2, conv_k=4) == 87 + 10
    assert bench.algorithmic_valu_slots(16, True, 2, flags=3, conv_k=4) == 87 + 56 + 10
    # backward, counted per variant: 16 N + 60 (Euler), 56 N + 60 (exact ZOH),
    # and 48 more per element with the conv prologue
    assert bench.bwd_valu_slots(16, True, 2) == 316
    assert bench.bwd_valu_slots(16, True, 2, flags=2) == 316
    assert bench.bwd_valu_slots(16, True, 2, flags=1) == 956
    assert bench.bwd_valu_slots(16, True, 2, flags=0, conv_k=4) == 364
    assert bench.bwd_valu_slots(16, True, 2, flags=3, conv_k=4) == 1004
    assert bench.bwd_valu_slots(16, True, 2, general_a=True) == 380
