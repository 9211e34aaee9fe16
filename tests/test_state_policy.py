"""The 8/32-bit state policy (host logic only, CPU)."""
import torch

from bit_optimizer_states_amd import state


def test_min_8bit_size_is_strict():
    # fewer than min_8bit_size elements -> 32-bit; exactly min_8bit_size -> 8-bit
    assert not state.uses_8bit(4095)
    assert state.uses_8bit(4096)
    assert not state.uses_8bit(16383, min_8bit_size=16384)
    assert state.uses_8bit(16384, min_8bit_size=16384)
    assert not state.uses_8bit(10 ** 9, force_32bit=True)


def test_allocate_shapes_and_fresh_values():
    params = [torch.zeros(4096), torch.zeros(100), torch.zeros(5000), torch.zeros(8192)]
    st = state.allocate(params, kind=0, blocksize=2048, min_8bit_size=4096, force_32bit={3})
    s1, s2, a1, a2 = st[0]
    assert s1.dtype == torch.uint8 and s1.numel() == 4096 and torch.all(s1 == 127) and torch.all(s2 == 127)
    assert a1.numel() == 2 and torch.all(a1 == 0) and a2.numel() == 2
    for k in (1, 3):                                   # too small; forced
        s1, s2, a1, a2 = st[k]
        assert s1.dtype == torch.float32 and torch.all(s1 == 0) and s2.dtype == torch.float32
        assert a1 is None and a2 is None
    s1, s2, a1, a2 = st[2]
    assert a1.numel() == 3                             # ceil(5000 / 2048)
    one = state.allocate(params, kind=2)               # Lion: one state
    assert all(s2 is None and a2 is None for (_, s2, _, a2) in one)
