"""What the sharp full-size parity variant can tell apart, shown with the oracle on the CPU.

With the workloads' own distributions (keys N(0,1)/sqrt(128), queries N(0,1)) the softmax
is nearly uniform and |out| ~ 0.088 / sqrt(L), about 5e-4 at 32,768 tokens: there an
output that attended wrong blocks can sit inside the 2e-3 gate. The sharp variant (queries x 32,
values N(0, 1)) makes outputs of order 1 built from a few tokens; there the relative gate
max |error| / max |out| of the GPU tests must reject the mistakes a paged kernel can make:
reading the second half of a text's blocks from the wrong place (an addressing error past
some offset), or dropping the block that holds a head's heaviest token. Mistakes are
planted in the oracle's inputs, on the CPU.
"""
import math

import numpy as np

import workloads as wl
from oracle.attention import softmax_attention

REL_GATE_F16 = 2.0 ** -11 + 1e-3  # as in test_gpu_workloads.REL_GATE["f16"]


def text0(w):
    """Keys, values and queries of the first text of workload w (one step): [L, H, D]."""
    d = wl.draw(w.scaled(num_seqs=1, steps=1))
    k = np.concatenate([d.prefill_k[0].double().numpy(), d.step_k[0].double().numpy()])
    v = np.concatenate([d.prefill_v[0].double().numpy(), d.step_v[0].double().numpy()])
    return k, v, d.step_q[0][0].double().numpy()


def outputs(k, v, q):
    D = q.shape[-1]
    return np.stack([softmax_attention(q[h], k[:, h], v[:, h], 1 / math.sqrt(D))
                     for h in range(q.shape[0])])


def rel(got, want):
    return float(np.abs(got - want).max() / np.abs(want).max())


def test_sharp_gate_sees_wrong_blocks():
    k, v, q = text0(wl.sharp(wl.OPT13B_7x2048))
    want = outputs(k, v, q)
    assert np.abs(want).max() > 0.5
    B, L = 16, k.shape[0]
    # the second half of the blocks read from the wrong place
    half = (L // B // 2) * B
    k2, v2 = k.copy(), v.copy()
    k2[half:], v2[half:] = k[:L - half][::-1], v[:L - half][::-1]
    assert rel(outputs(k2, v2, q), want) > 20 * REL_GATE_F16
    # the block holding head 0's heaviest token dropped
    z = k[:, 0] @ q[0]
    b = int(np.argmax(z)) // B
    keep = np.r_[0:b * B, min(L, (b + 1) * B):L]
    assert rel(outputs(k[keep], v[keep], q), want) > 20 * REL_GATE_F16
