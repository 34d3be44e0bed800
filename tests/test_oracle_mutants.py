"""Planted-mistake tests: every plausible slip in the oracle must trip a pin.

Each case rewrites one line of the oracle's source (on the CPU, in a private
module object), runs the pin checks of ``test_oracle_pins`` against the
mutated copy, and requires at least one of them to fail.  This is what shows
that the pins constrain the oracle (a dropped term, a wrong sign, a wrong
index or a transposed operand cannot survive them).
"""
import os
import types

import pytest

import test_oracle_pins as pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

MUTATIONS = [
    # (id, file, original text, planted mistake)
    ("gqa_modulo_mapping", "attention.py",
     "heads = q64[b, g * G:(g + 1) * G, :]", "heads = q64[b, g::Hkv, :]"),
    ("block_slot_swapped", "attention.py",
     "phys = np.asarray(block_tables)[b, t // bs]", "phys = np.asarray(block_tables)[b, t % bs]"),
    ("scale_dropped", "attention.py",
     "logits = s * (K[:, g, :] @ heads.T)", "logits = (K[:, g, :] @ heads.T)"),
    ("normaliser_over_all_heads", "attention.py",
     "w.sum(axis=0)[:, None]", "w.sum()"),
    ("weights_times_keys", "attention.py",
     "(w.T @ V[:, g, :])", "(w.T @ K[:, g, :])"),
    ("query_of_first_sequence", "attention.py",
     "heads = q64[b, g * G:(g + 1) * G, :]", "heads = q64[0, g * G:(g + 1) * G, :]"),
    ("context_off_by_one", "attention.py",
     "K = upcast(gather_sequence(k_cache, block_tables, b, n), dtype)  # [n, Hkv, D]",
     "K = upcast(gather_sequence(k_cache, block_tables, b, n), dtype)  # [n, Hkv, D]\n"
     "        n = n - 1 if n > 1 else n; K = K[:n]; V = upcast(gather_sequence(v_cache, "
     "block_tables, b, n), dtype)"),
    ("phase2_rescale_dropped", "attention.py",
     "rescale = np.exp(m - global_max) * s", "rescale = s"),
    ("phase2_rescale_sign", "attention.py",
     "rescale = np.exp(m - global_max) * s", "rescale = np.exp(global_max - m) * s"),
    ("phase2_expsum_dropped", "attention.py",
     "rescale = np.exp(m - global_max) * s", "rescale = np.exp(m - global_max)"),
    ("partial_not_normalised", "attention.py",
     "return m, ssum, (e @ V) / ssum", "return m, ssum, (e @ V)"),
    ("partition_range_off_by_one", "attention.py",
     "lo, hi = p * P, min((p + 1) * P, n)", "lo, hi = p * P, min((p + 1) * P, n - 1)"),
    ("partition_count_floor", "attention.py",
     "return (int(n) + int(partition_size) - 1) // int(partition_size)",
     "return max(int(n) // int(partition_size), 1)"),
    ("bf16_shift_wrong", "storage.py",
     "word = a.astype(np.uint32) << np.uint32(16)", "word = a.astype(np.uint32) << np.uint32(15)"),
    ("f16_read_as_bf16", "storage.py",
     "return a.astype(np.float64)\n    if dtype == \"bf16\"",
     "return a.view(np.uint16).astype(np.float64)\n    if dtype == \"bf16\""),
]


def _load(name, src_override=None):
    path = os.path.join(ORACLE_DIR, name)
    src = open(path).read() if src_override is None else src_override
    return src


def build_mutant(fname, old, new):
    srcs = {f: _load(f) for f in ("storage.py", "attention.py")}
    assert srcs[fname].count(old) >= 1, f"mutation target not found in {fname}: {old!r}"
    srcs[fname] = srcs[fname].replace(old, new, 1)
    st = types.ModuleType("mutant_storage")
    exec(compile(srcs["storage.py"], "mutant_storage.py", "exec"), st.__dict__)
    at = types.ModuleType("mutant_attention")
    at_src = srcs["attention.py"].replace("from .storage import upcast", "upcast = _upcast")
    at.__dict__["_upcast"] = st.upcast
    exec(compile(at_src, "mutant_attention.py", "exec"), at.__dict__)
    return at, st


@pytest.mark.parametrize("mid,fname,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(mid, fname, old, new):
    at, st = build_mutant(fname, old, new)
    failures = []
    for check in pins.ALL_CHECKS:
        try:
            check(at)
        except Exception as exc:  # any assertion or crash counts as caught
            failures.append((check.__name__, type(exc).__name__))
    assert failures, f"planted mistake {mid} survived every pin"


def test_unmutated_copy_passes_every_pin():
    at, st = build_mutant("attention.py", "import math", "import math")
    for check in pins.ALL_CHECKS:
        check(at)
