"""A seeded random sweep of shapes and options through selscan_fwd_ex and
selscan_bwd_ex against the fp64 oracle.

Each case draws the batch, length and channel count (so that lanes past dim,
ragged tails, one or many sequence parts all occur), the state size, the
I/O type, the gate and h0, the kind of A (S4D-real: the power chain;
perturbed: the per-(t, n) exponential; mixed: both kinds of channel group in
one call), the direction, exact zero-order hold and the conv prologue's
width, then checks the forward's y and h_last and every gradient of the
backward against the oracle with the usual tolerances.  The sizes are capped
so that the oracle takes well under a second per case.
"""
import numpy as np
import pytest

import selscan_inputs as si
import selective_state_space_selscan_amd as ss
import test_parity_bwd_variants as bv
import test_parity_variants as fv

pytestmark = pytest.mark.gpu

ZOH = ss.SELSCAN_FLAG_ZOH_EXACT
REV = ss.SELSCAN_FLAG_REVERSE


def draw_cases(count=32, seed=9100):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(count):
        N = int(rng.choice([4, 8, 16, 32, 64]))
        batch = int(rng.integers(1, 4))
        if k % 2 == 0:
            # log-uniform: tiny and ragged sizes
            dim = int(np.exp(rng.uniform(0.0, np.log(300.0))))
            L = int(np.exp(rng.uniform(0.0, np.log(1400.0))))
        else:
            dim = int(rng.integers(1, 300))
            L = int(rng.integers(1, 1400))
        while batch * L * dim * N > 12_000_000 and L > 1:
            L = max(1, L // 2)
        out.append(dict(
            k=k, N=N, batch=batch, dim=dim, L=L,
            dtype=si.F32 if rng.random() < 0.4 else si.BF16,
            gate=bool(rng.random() < 0.7), h0=bool(rng.random() < 0.5),
            A=str(rng.choice(["s4d", "perturbed", "mixed"])),
            flags=int(rng.choice([0, REV, ZOH, ZOH | REV])),
            conv=int(rng.choice([0, 0, 1, 2, 3, 4])),
            seed=9200 + 10 * k))
    return out


CASES = draw_cases()


def case_id(c):
    return "%d-b%dL%dd%dN%d-%s-%s-f%d-c%d" % (c["k"], c["batch"], c["L"], c["dim"], c["N"],
                                              c["dtype"], c["A"], c["flags"], c["conv"])


@pytest.mark.parametrize("case", CASES, ids=[case_id(c) for c in CASES])
def test_sweep_forward_and_backward(device, case):
    c = case
    print("sweep case", case_id(c), flush=True)
    inp = si.make_fwd_inputs(c["batch"], c["L"], c["dim"], c["N"], c["dtype"], c["gate"],
                             seed=c["seed"], h0=c["h0"])
    if c["A"] == "perturbed":
        inp.A = si.perturbed_A(c["dim"], c["N"], c["seed"] + 1)
    elif c["A"] == "mixed":
        inp.A = si.mixed_A(c["dim"], c["N"], c["seed"] + 1)
    conv = None if c["conv"] == 0 else si.conv_params(c["dim"], c["conv"], c["seed"] + 2)
    fv.check_ex(inp, device, c["flags"], conv, what="sweep")
    bv.check_bwd_ex(inp, device, c["seed"] + 3, c["flags"], conv, what="sweep")
