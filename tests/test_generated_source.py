"""The committed attention loop block (csrc/attn_loop.inc) is exactly what
csrc/gen_attn_loop.py writes, so the generator stays the source of truth."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "item_scoring_attention_amd", "csrc")


def _generator():
    spec = importlib.util.spec_from_file_location("gen_attn_loop", os.path.join(CSRC, "gen_attn_loop.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_attn_loop_inc_matches_generator():
    with open(os.path.join(CSRC, "attn_loop.inc")) as f:
        committed = f.read()
    assert committed == _generator().render()


def test_loop_block_waits_fit_the_counter():
    # every LDS wait of the generated block fits lgkmcnt's 4-bit field, and
    # every label is per-instance (%=) so two inlined copies never clash
    text = _generator().render()
    for tok in text.split("lgkmcnt(")[1:]:
        assert int(tok.split(")")[0]) <= 15
    for ln in text.splitlines():
        if ln.strip().startswith('"L') and ln.strip().endswith(':\\n" \\'):
            assert ln.strip().startswith('"L%=_')
