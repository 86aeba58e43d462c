"""GPU behaviour on special values: a NaN in the input propagates exactly as
in the recurrence, and nowhere else.

A NaN at u[b, t0, d] makes the state of channel (b, d) NaN from step t0 on
(through the sequence-part boundaries: the part summaries and the carried
entry states), hence y[b, t >= t0, d] and h_last[b, d, :] in the forward
direction; every other channel and every earlier step is unaffected.  The
oracle, a plain sequential loop, shows the same pattern; both are compared
where finite.
"""
import numpy as np
import pytest
import torch

import oracle
import selscan_inputs as si
import selective_state_space_selscan_amd as ss
from parity_util import TOL, rel_err, to_np

pytestmark = pytest.mark.gpu

ZOH, REV = ss.SELSCAN_FLAG_ZOH_EXACT, ss.SELSCAN_FLAG_REVERSE


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("flags,conv", [(0, False), (ZOH | REV, True)], ids=["plain", "zoh_rev_conv"])
def test_nan_propagates_like_the_recurrence(device, flags, conv):
    inp = si.make_fwd_inputs(2, 777, 130, 16, si.BF16, True, seed=1700, h0=True)
    b0, t0, d0 = 1, 400, 70
    inp.u.value[b0, t0, d0] = np.nan
    inp.u.bits[b0, t0, d0] = 0x7FC0   # bf16 quiet NaN
    say("case nan", flags, conv)
    cw, cb = si.conv_params(130, 4, 1701) if conv else (None, None)
    t = si.fwd_tensors(inp, device)
    y, hL = ss.selscan_fwd_ex(t["u"], t["delta"], t["A"], t["Bm"], t["Cm"], t["D_skip"], t["z"],
                              t["delta_bias"], True, t["h0"], return_last_state=True, flags=flags,
                              conv_weight=None if cw is None else torch.from_numpy(cw).to(device),
                              conv_bias=None if cb is None else torch.from_numpy(cb).to(device))
    torch.cuda.synchronize()
    ey, eh = oracle.fwd(inp.u.value, inp.delta.value, inp.A, inp.Bm.value, inp.Cm.value,
                        inp.D_skip, inp.z.value, inp.delta_bias, True, inp.h0, flags=flags,
                        conv_w=cw, conv_b=cb)
    gy, gh = to_np(y), to_np(hL)
    # the expected pattern: channel (b0, d0) from t0 on in scan order
    mask = np.zeros(ey.shape, bool)
    if flags & REV:
        mask[b0, :t0 + 1, d0] = True
    else:
        mask[b0, t0:, d0] = True
    assert np.array_equal(np.isnan(ey), mask), "oracle NaN pattern"
    assert np.array_equal(np.isnan(gy), mask), "kernel NaN pattern"
    hmask = np.zeros(eh.shape, bool)
    hmask[b0, d0, :] = True
    assert np.array_equal(np.isnan(eh), hmask) and np.array_equal(np.isnan(gh), hmask)
    ok = ~mask
    ry = rel_err(gy[ok], ey[ok])
    rh = rel_err(gh[~hmask], eh[~hmask])
    say("  rel_err elsewhere y=%.3g h_last=%.3g" % (ry, rh))
    assert ry <= TOL[si.BF16] and rh <= TOL[si.BF16]
