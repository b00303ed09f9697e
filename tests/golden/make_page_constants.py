"""Writes page_constants.json: closed-form read-outs of the L2 norm and scale.

The values follow from two constants stated on the pages, not from any code:
  * the L2 norm adds eps = 1e-6 to the sum of squares under the square root
    (KdaTcVerify, page "vllm.models.kimi_k3.nvidia.recoverssm.cutedsl.verify",
    the norm step of the kernel);
  * chunk_kda's default scale is 128^-0.5 (page "mate.kda", chunk_kda).
With a zero write strength, no decay and an identity start state, the output of
one token is scale * q / sqrt(sum(q^2) + eps), channel by channel.  Inputs are
powers of two or small integers, exact in fp32.
"""
import json
import math
import os

EPS = 1e-6
cases = []


def case(name, q, scale):
    s = sum(x * x for _, x in q)
    sc = 128 ** -0.5 if scale is None else scale
    out = [[i, sc * x / math.sqrt(s + EPS)] for i, x in q]
    cases.append(dict(name=name, q=q, scale=scale, o=out))


case("tiny_norm_default_scale", [[3, 2.0 ** -13]], None)
case("pythagorean_unit_scale", [[0, 3.0], [1, 4.0]], 1.0)
case("eps_dominated", [[0, 2.0 ** -20], [127, -(2.0 ** -21)]], 1.0)
case("large_norm_default_scale", [[5, 1024.0], [6, -2048.0], [100, 0.5]], None)

with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "page_constants.json"), "w") as f:
    json.dump(dict(source="closed forms of the L2-norm eps and the default scale; "
                          "see make_page_constants.py", cases=cases), f, indent=1)
