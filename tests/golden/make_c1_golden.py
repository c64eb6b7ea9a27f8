"""Write c1_expected_selection.npz from the oracle alone (a regression record).

Run from the repository root:  python tests/golden/make_c1_golden.py
It calls only ``oracle`` and ``workload``.
"""
import sys
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parents[2]
sys.path.insert(0, str(ROOT))

import oracle  # noqa: E402
import workload as W  # noqa: E402


def main():
    s = W.CONFIGS["c1_8k_gqa8"]
    q = W.gen_q(s)
    kv = W.gen_kv(s)
    lab = W.label_channels(s, kv[0])
    st = oracle.decode(s, q, kv, lab)
    np.savez_compressed(Path(__file__).with_name("c1_expected_selection.npz"), label_ch=lab,
                        S=st.S, block_idx=st.block_idx, token_idx=st.token_idx, out=st.out, lse=st.lse)


if __name__ == "__main__":
    main()
