"""Host-side checks of the build/smoke entry module (no GPU needed)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402


def test_smoke_configs_build_inputs():
    import __graft_entry__ as ge
    f32, bf16, dec = ge.smoke_configs()
    assert (f32.dtype, bf16.dtype, dec.dtype) == ("f32", "bf16", "bf16")
    assert dec.mode == "decode" and dec.kv_len <= dec.S
    for cfg in (f32, bf16):
        inp = synth.make_prefill_inputs(cfg)
        assert tuple(inp["q"].shape) == (cfg.B, cfg.S, cfg.N + 1, cfg.d)
    inp = synth.make_decode_inputs(dec)
    assert tuple(inp["k"].shape) == (dec.B, dec.G, dec.S, dec.d)
    assert int(inp["kv_len"][0]) == dec.kv_len
