"""Planted mistakes in copies of the oracle must be caught by the pins.

Each mutant is a fresh copy of oracle/sfa.py with one plausible error (a
dropped term, a wrong sign or index, a transposed operand). The copy is
loaded under its own module name, so the real oracle is untouched.
"""
import importlib.util
import pathlib

import numpy as np
import pytest

from oracle_pins import ALL_PINS

SRC = pathlib.Path(__file__).resolve().parent.parent / "oracle" / "sfa.py"

MUTANTS = {
    # causal mask leaks one future position
    "causal_off_by_one": ("allowed = Q <= P\n", "allowed = Q <= P + 1\n"),
    # window admits W+1 keys
    "window_inclusive": ("allowed &= (P - Q) < window", "allowed &= (P - Q) <= window"),
    # intra compares tokens instead of streams
    "intra_token_not_stream": ("allowed &= (Q % n) == (P % n)", "allowed &= (Q // n) == (P // n)"),
    # stream-major placement instead of token-major
    "interleave_stream_major": ("out[:, k::n] = src[k]", "out[:, k * L:(k + 1) * L] = src[k]"),
    # GQA maps heads round-robin
    "gqa_round_robin": ("kh = h // G\n                ob", "kh = h % Hkv\n                ob"),
    # softmax scale dropped
    "no_scale": ("s = float(scale) * (q @ k.T)", "s = (q @ k.T)"),
    # values replaced by keys (transposed/wrong operand)
    "pv_uses_keys": ("o = (w @ v) / den", "o = (w @ k) / den"),
    # lse without the max term
    "lse_no_max": ("lse = m[:, 0] + np.log(den[:, 0])", "lse = np.log(den[:, 0])"),
    # decode queries one position too early
    "decode_rows_shift": ("rows = (T - 1) * n + np.arange(n)", "rows = (T - 1) * n + np.arange(n) - 1"),
    # last-stream queries placed at stream 0 instead of stream n-1
    "last_stream_at_stream0": ("rows = np.arange(L) * n + (n - 1)", "rows = np.arange(L) * n"),
    # embedding rows taken from table 0 for every stream
    "embed_one_table": ("per_stream[k][valid] = tables[k][ids[valid]]", "per_stream[k][valid] = tables[0][ids[valid]]"),
    # rotation in the wrong direction
    "rope_sign": ("[a * c - b * s, b * c + a * s]", "[a * c + b * s, b * c - a * s]"),
    # rotary frequencies with exponent 2j/half instead of 2j/d
    "rope_freq": ("theta = base ** (-2.0 * np.arange(half, dtype=np.float64) / d)",
                  "theta = base ** (-2.0 * np.arange(half, dtype=np.float64) / half)"),
    # paged cache: every stream reads stream 0's pages
    "paged_stream0_table": ("pages[bt[k, t // P], t % P]", "pages[bt[0, t // P], t % P]"),
    # paged cache: row within the page off by one
    "paged_row_shift": ("pages[bt[k, t // P], t % P]", "pages[bt[k, t // P], (t + 1) % P]"),
    # per-sequence lengths ignored: every sequence decodes at the first one's length
    "paged_one_length": ("T = int(seq_lens[b])", "T = int(seq_lens[0])"),
    # backward: dS without the rowsum correction
    "bwd_no_rowsum": ("ds = pr * (dp - (dp * pr).sum(axis=1, keepdims=True))", "ds = pr * dp"),
    # backward: dK built from dP instead of dS
    "bwd_dk_from_dp": ("dk[b, :, kh] += float(scale) * (ds.T @ q[b, rr, h])",
                       "dk[b, :, kh] += float(scale) * (dp.T @ q[b, rr, h])"),
    # decode reads one token too many from the cache
    "decode_reads_future": ("[:, :, :T]\n    vc", "[:, :, :T + 1]\n    vc"),
}


def _load_mutant(name, old, new):
    text = SRC.read_text()
    assert text.count(old) == 1, f"mutation site for {name} not unique"
    spec = importlib.util.spec_from_loader(f"oracle_mutant_{name}", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(text.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    mod = _load_mutant(name, old, new)
    caught = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutant {name} passed every pin"
