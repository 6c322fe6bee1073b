"""The watchdog path: a watchdog of (almost) zero length makes the first wait that is not
already satisfied give up; the launch must still end, report the timeout in the status word,
and the next step must refuse with AMK_E_DEVICE_TIMEOUT."""
import os
import pytest
import torch

import amk_inputs as I


@pytest.mark.gpu
def test_watchdog_timeout_ends_launch_and_is_reported(monkeypatch):
    import persistent_megakernel_amd as M
    # two SmolLM2-shaped layers: the O projection waits several microseconds for attention,
    # so its first poll finds no data and the (almost) zero watchdog expires there
    shape = I.SHAPES["smollm2_135m_bf16"].replace(n_layers=2)
    w = I.make_weights(shape)
    toks = torch.zeros(4, dtype=torch.int32, device="cuda")
    monkeypatch.setenv("AMK_WATCHDOG_MS", "1e-6")   # read when the context is created
    dec = M.Decoder(shape, w)
    dec.step(toks[0:1], 0, toks[1:2])
    torch.cuda.synchronize()
    st = dec.status()
    print("status after the short watchdog:", st, flush=True)
    assert st & M.STATUS_TIMEOUT
    with pytest.raises(M.AmkError) as ei:
        dec.step(toks[1:2], 1, toks[2:3])
    assert ei.value.status == M._abi.AMK_E_DEVICE_TIMEOUT
    dec.close()
    # a new context with the normal watchdog runs normally
    monkeypatch.delenv("AMK_WATCHDOG_MS")
    dec = M.Decoder(shape, w)
    dec.step(toks[0:1], 0, toks[1:2])
    torch.cuda.synchronize()
    assert dec.status() == 0
    dec.close()
