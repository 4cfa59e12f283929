"""Bounded waits inside the persistent kernels.  Every wait ends by
construction; each is also bounded in time, and one that gives up is recorded
on the device and reported by moe_sync_status as MOE_ETIMEOUT while the
kernel still runs to its end.  The give-up path is forced from the host
(MOE_DEBUG_UNREACHABLE_WAITS: every wait targets one more than can happen,
MOE_WAIT_LIMIT_US=0: give up at once; both read by moe_init), so every kernel
exits normally."""

import pytest
import torch

import synth
import combine_moe_route_histogram_amd as M
from combine_moe_route_histogram_amd import layer as L
from gpu_util import custom_config, debug_settings, device_inputs

pytestmark = pytest.mark.gpu

OUTS = ("out", "y", "dab", "dx_rows", "dx", "dw1", "dw2")


def _setup():
    cfg = custom_config(300, 256, 8, 2, 320, 0, "bf16", number=500)
    p = device_inputs(synth.make_inputs(cfg, with_grad=True))
    d = L.make_dims(cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, 0, "bf16")
    return d, p


def _step(b, p, fused):
    L.forward(b, p, fused=fused)
    L.backward(b, p, fused=fused)


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "plain"])
def test_forced_timeout_is_reported_then_cleared(fused):
    print(f"case forced wait timeout fused={fused}", flush=True)
    d, p = _setup()
    b = L.Buffers(d)
    _step(b, p, fused)
    M.moe_sync_status()                      # a normal step records nothing
    ref = {n: getattr(b, n).clone() for n in OUTS}

    with debug_settings(MOE_DEBUG_UNREACHABLE_WAITS=1, MOE_WAIT_LIMIT_US=0):
        _step(b, p, fused)                   # kernels give up their waits and exit
        with pytest.raises(M.MoeError) as err:
            M.moe_sync_status()
        assert err.value.status == 5         # MOE_ETIMEOUT
        M.moe_sync_status()                  # the record was cleared

    _step(b, p, fused)
    M.moe_sync_status()
    for n, t in ref.items():
        assert torch.equal(t, getattr(b, n)), n
