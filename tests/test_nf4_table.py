"""The library's NF4 level table (generated at build time by bisection on the
normal CDF) against the oracle's (scipy's normal quantile function): two
independent computations of the same definition must give the same fp16
bits, and the header the kernels compile must be the generator's output."""

import os
import re

import numpy as np

from conftest import ROOT


def test_library_table_matches_oracle(oracle_mod):
    import oracle.nf4 as onf4
    from bit_weight_only_wq_amd import gen_nf4
    bits = [b for b, _ in gen_nf4.levels()]
    assert bits == [int(v) for v in onf4.levels().view(np.uint16)]
    # The committed header is what the generator writes now.
    text = open(os.path.join(ROOT, "bit_weight_only_wq_amd", "csrc", "wq_nf4_levels.h")).read()
    assert text == gen_nf4.render()
    got = [int(x, 16) for x in re.search(r"kNf4LevelBits\[16\] = \{([^}]*)\}", text).group(1).split(",")]
    assert got == bits
    mids = [float.fromhex(x.strip().rstrip("f")) for x in
            re.search(r"kNf4Mid\[15\] = \{([^}]*)\}", text).group(1).split(",")]
    assert np.array_equal(np.array(mids, dtype=np.float32), onf4.midpoints())
