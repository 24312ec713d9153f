"""Plant plausible mistakes in copies of the oracle (CPU only) and show that
the pin battery rejects every one of them.  The oracle source itself is never
modified: each mutant is a textual edit of a temporary copy, compiled with the
same flags."""
import os

import pytest

import oracle as O
import pins

MUTANTS = {
    "no_error_feedback": ("acc[i] = grad[a + i] + residual[a + i];",
                          "acc[i] = grad[a + i];"),
    "ties_to_high_index": [("| (uint64_t)(0xffffffffu - (uint32_t)i);",
                            "| (uint64_t)((uint32_t)i);"),
                           ("chosen[j] = 0xffffffffu - (uint32_t)(word[j] & 0xffffffffu);",
                            "chosen[j] = (uint32_t)(word[j] & 0xffffffffu);")],
    "signed_order": ("return u & 0x7fffffffu;", "return u ^ 0x80000000u;"),
    "sent_residual_kept": ("residual[a + li] = 0.0f;", "residual[a + li] = acc[li];"),
    "k_floor": ("__int128 q = (p + (den - 1)) / den;", "__int128 q = p / den;"),
    "local_index": ("msg_idx[mpos + j] = (uint32_t)(a + li);",
                    "msg_idx[mpos + j] = (uint32_t)(li);"),
    "drop_worker0": ("for (int32_t p = 0; p < P; ++p) {", "for (int32_t p = 1; p < P; ++p) {"),
    "sum_not_mean": ("float s = lr / (float)P;", "float s = lr;"),
    "reverse_worker_order": ("for (int32_t p = 0; p < P; ++p) {",
                             "for (int32_t p = P - 1; p >= 0; --p) {"),
    "fused_update": ("float d = s * u[i];\n        w[i] = w[i] - d;",
                     "w[i] = __builtin_fmaf(-s, u[i], w[i]);"),
    "unsorted_message": ("qsort(chosen, (size_t)kl, sizeof(uint32_t), asc_u32);", ""),
}


def _battery(o):
    failures = []
    for pin in pins.ALL_FAST_PINS:
        try:
            pin(o)
        except AssertionError:
            failures.append(pin.__name__)
    return failures


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    edits = MUTANTS[name]
    if isinstance(edits, tuple):
        edits = [edits]
    src = open(O.SRC).read()
    for old, new in edits:
        assert src.count(old) == 1, f"mutation site for {name} not unique"
        src = src.replace(old, new)
    path = os.path.join(tmp_path, f"mut_{name}.c")
    with open(path, "w") as f:
        f.write(src)
    lib = O.build(src=path, out=os.path.join(tmp_path, f"libmut_{name}.so"))
    caught = _battery(O.Oracle(lib))
    assert caught, f"mutant {name} passed every pin"
