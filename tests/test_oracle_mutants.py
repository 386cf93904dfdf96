"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that a pin catches each.

Every mutant is the oracle's own source with one edit; a mutant that passed
every pin would mean the pins cannot tell that mistake from the truth.
"""
import importlib.util
import os
import shutil
import sys
import uuid

import pytest

from tests import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "exclusive_causal_diagonal": ("attention.py", "causal = k_pos[None, :] <= q_pos[:, None]",
                                  "causal = k_pos[None, :] < q_pos[:, None]"),
    "doc_mask_not_equality": ("attention.py", "(k_doc[None, :] == q_doc[:, None])",
                              "(k_doc[None, :] <= q_doc[:, None])"),
    "scale_one_over_d": ("attention.py", "    if scale is None:\n        scale = 1.0 / math.sqrt(d)\n    o = ",
                         "    if scale is None:\n        scale = 1.0 / d\n    o = "),
    "gqa_head_modulo": ("attention.py", "return (h * hkv) // hq", "return h % hkv"),
    "lse_drops_max": ("attention.py", "np.where(has, m_safe + np.log(", "np.where(has, np.log("),
    "ds_sign": ("attention.py", "ds = p * (dp - delta[:, None])", "ds = p * (dp + delta[:, None])"),
    "dk_unscaled": ("attention.py", "dk[b, kh] += scale * (ds.T @ q[b, h, rows])",
                    "dk[b, kh] += (ds.T @ q[b, h, rows])"),
    "dp_wrong_operand": ("attention.py", "dp = do[b, h, rows] @ vc.T", "dp = do[b, h, rows] @ kc.T"),
    "dv_uses_ds": ("attention.py", "dv[b, kh] += p.T @ do[b, h, rows]", "dv[b, kh] += ds.T @ do[b, h, rows]"),
    "dq_uses_p": ("attention.py", "dq[b, h, rows] = scale * (ds @ kc)", "dq[b, h, rows] = scale * (p @ kc)"),
    "merge_max_not_logaddexp": ("ring.py", "lse = np.logaddexp(lse_a, lse_b)", "lse = np.maximum(lse_a, lse_b)"),
    "merge_weight_swapped": ("ring.py", "o = w_a[..., None] * o_a + w_b[..., None] * o_b",
                             "o = w_b[..., None] * o_a + w_a[..., None] * o_b"),
    "local_block_counted_twice": ("ring.py", "order = [(r - t) % n for t in range(n)]",
                                  "order = [r] + [(r - t) % n for t in range(n)]"),
    "zigzag_wrong_mirror": ("ring.py", "np.arange((2 * n - 1 - r) * c, (2 * n - r) * c)",
                            "np.arange((2 * n - 2 - r) * c, (2 * n - 1 - r) * c)"),
    "softmax_no_normalise": ("attention.py", "p = e / np.where(has, l, 1.0)[:, None]", "p = e"),
}


def _load_mutant(tmp_path, name):
    fname, old, new = MUTANTS[name]
    pkg = f"oracle_mutant_{name}_{uuid.uuid4().hex[:8]}"
    dst = tmp_path / pkg
    shutil.copytree(os.path.join(ROOT, "oracle"), dst)
    src = (dst / fname).read_text()
    assert src.count(old) >= 1, f"mutation site missing: {name}"
    (dst / fname).write_text(src.replace(old, new, 1))
    spec = importlib.util.spec_from_file_location(pkg, dst / "__init__.py",
                                                  submodule_search_locations=[str(dst)])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[pkg] = mod
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_a_pin_catches_the_mutant(tmp_path, name):
    mutant = _load_mutant(tmp_path, name)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except Exception as e:      # AssertionError, or the mutant crashing on a shape
            caught.append((pin.__name__, type(e).__name__))
            break
    assert caught, f"no pin detects mutant {name}"
