"""The seeded input recipe: the same seed gives the same tensors bit for bit,
optional parts do not shift the other draws, and the drawn values have the
recipe's structure (softplus(bias) = dt in [1e-3, 1e-1], A = -(n+1), bf16 =
round-to-nearest-even of the fp32 draw)."""
from __future__ import annotations

import numpy as np
import torch

from workloads import decode_inputs, inverse_softplus, scan_inputs, workload_inputs


def _same(p, q):
    assert p.keys() == q.keys()
    for k in p:
        if isinstance(p[k], torch.Tensor):
            assert torch.equal(p[k], q[k]), k
        else:
            assert p[k] == q[k], k


def test_same_seed_same_tensors():
    _same(workload_inputs(0), workload_inputs(0))
    _same(scan_inputs(2, 33, 16, 4, torch.bfloat16, seed=5), scan_inputs(2, 33, 16, 4, torch.bfloat16, seed=5))
    _same(decode_inputs(3, 16, 8, 2, seed=1), decode_inputs(3, 16, 8, 2, seed=1))
    a, b = scan_inputs(1, 20, 8, 4, seed=1), scan_inputs(1, 20, 8, 4, seed=2)
    assert not torch.equal(a["u"], b["u"])


def test_optional_parts_do_not_shift_other_draws():
    full = scan_inputs(2, 40, 16, 4, seed=3)
    bare = scan_inputs(2, 40, 16, 4, seed=3, with_z=False, with_D=False, with_bias=False)
    for k in ("u", "delta", "B", "C", "A"):
        assert torch.equal(full[k], bare[k]), k
    assert bare["z"] is None and bare["D"] is None and bare["delta_bias"] is None


def test_recipe_structure():
    p = scan_inputs(1, 10, 512, 16, seed=0)
    dt = np.logaddexp(0.0, p["delta_bias"].double().numpy())
    assert dt.min() >= 1e-3 * (1 - 1e-5) and dt.max() <= 1e-1 * (1 + 1e-5)
    assert torch.equal(p["A"], -torch.arange(1, 17, dtype=torch.float32).expand(512, 16))
    x = torch.tensor([1e-3, 1e-2, 0.05])
    assert torch.allclose(torch.nn.functional.softplus(inverse_softplus(x).double()), x.double(),
                          rtol=1e-6)


def test_bf16_is_the_rounded_fp32_draw():
    p32 = scan_inputs(2, 30, 24, 8, torch.float32, seed=9)
    p16 = scan_inputs(2, 30, 24, 8, torch.bfloat16, seed=9)
    for k in ("u", "delta", "z", "B", "C"):
        assert torch.equal(p32[k].to(torch.bfloat16), p16[k]), k
    for k in ("A", "D", "delta_bias"):
        assert torch.equal(p32[k], p16[k]), k
