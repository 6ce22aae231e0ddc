"""The binding's checks of caller-supplied outputs (no GPU needed: the checks run
before any library call).  The library sizes every write from the shape
arguments, so an output of the wrong shape, dtype, layout or device must be
refused with an exception, never passed on as a raw pointer."""
import numpy as np
import pytest
import torch

from exact_attention_85_amd import _binding as b

CPU = torch.device("cpu")
SHAPE = (2, 3, 5, 64)


def test_accepts_an_exact_output():
    t = torch.empty(SHAPE, dtype=torch.bfloat16)
    assert b._check_out(t, "out", SHAPE, torch.bfloat16, CPU) is t


@pytest.mark.parametrize("bad", [
    torch.empty(SHAPE, dtype=torch.float32),                                 # dtype
    torch.empty((2, 3, 4, 64), dtype=torch.bfloat16),                        # too few rows
    torch.empty((2, 3, 5, 128), dtype=torch.bfloat16),                       # too wide
    torch.empty((2, 3, 64, 5), dtype=torch.bfloat16).transpose(2, 3),        # not contiguous
    torch.empty((2 * 3 * 5 * 64,), dtype=torch.bfloat16),                    # right size, wrong shape
])
def test_rejects_wrong_output(bad):
    with pytest.raises(ValueError):
        b._check_out(bad, "out", SHAPE, torch.bfloat16, CPU)


def test_rejects_other_device_and_non_tensor():
    t = torch.empty(SHAPE, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        b._check_out(t, "out", SHAPE, torch.bfloat16, torch.device("meta"))
    with pytest.raises(TypeError):
        b._check_out(np.empty(SHAPE, dtype=np.float32), "out", SHAPE, torch.bfloat16, CPU)


def test_outputs_allocates_or_checks_both():
    o, lse = b._outputs(None, None, 2, 3, 5, 64, CPU)
    assert o.shape == SHAPE and o.dtype == torch.bfloat16 and lse.shape == (2, 3, 5) and lse.dtype == torch.float32
    with pytest.raises(ValueError):
        b._outputs(o, torch.empty((2, 3, 5), dtype=torch.float64), 2, 3, 5, 64, CPU)
    with pytest.raises(ValueError):
        b._outputs(o, torch.empty((2, 3, 6), dtype=torch.float32), 2, 3, 5, 64, CPU)


def test_inputs_must_live_on_the_gpu():
    # the public entry points refuse host tensors before reaching the library
    q = torch.zeros(SHAPE, dtype=torch.bfloat16)
    for fn in (lambda: b.forward(q, q, q), lambda: b.forward_splitkv(q, q, q, num_splits=2),
               lambda: b.forward_window(q, q, q, 3, 0)):
        with pytest.raises(ValueError):
            fn()
