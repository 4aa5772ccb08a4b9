"""Writes rope_d2_closed_form.json: a hand-derivable d = 2 case.

With d = 2 there is one rotation pair and one frequency, theta^0 = 1, so a
vector at angle alpha with length rho, seen by a query at position t from a key
at logical position p, contributes rho_q * rho_k * cos(alpha_k - alpha_q + (p - t))
to the dot product of the rotated vectors (rotations compose by adding angles;
only the relative position p - t survives).  That is the score equation of the
MiniPIC page (section 2.1) evaluated in polar form, a different route from
rotating each vector with its own cos/sin pair.  The expected values below use
only this polar form and the definition of softmax; nothing here calls the
oracle or the HIP library.
"""
import json
import math
import os

# Inputs are exactly representable in bf16.
q = (1.0, 0.0)                 # query, angle 0, length 1
t = 3                          # its logical position
keys = [                       # (k0, k1, logical position)
    ((1.0, 0.0), 1),
    ((0.0, 1.0), 2),
    ((0.5, 0.5), 3),
    ((1.0, 0.0), 4),           # after the query: invisible
    ((-2.0, 0.0), -1),         # empty slot: invisible
]
values = [(0.25, -1.0), (2.0, 0.5), (-0.75, 1.5), (8.0, 8.0), (9.0, 9.0)]
scale = 1.0 / math.sqrt(2.0)


def polar(v):
    return math.hypot(v[0], v[1]), math.atan2(v[1], v[0])


rq, aq = polar(q)
scores, vis = [], []
for k, p in keys:
    rk, ak = polar(k)
    visible = 0 <= p <= t
    vis.append(visible)
    scores.append(rq * rk * math.cos(ak - aq + (p - t)) * scale if visible else None)
m = max(s for s in scores if s is not None)
z = sum(math.exp(s - m) for s in scores if s is not None)
prob = [math.exp(s - m) / z if s is not None else 0.0 for s in scores]
out = [sum(prob[j] * values[j][i] for j in range(len(keys))) for i in range(2)]
doc = {
    "citation": "MiniPIC (gist.science 2606.13126), section 2.1: score(t,j) = (R_t q_t)^T (R_pi(j) k_j) / sqrt(d); "
                "softmax attention over the visible keys; visibility 0 <= pi(j) <= t.",
    "derivation": __doc__.strip(),
    "theta": 10000.0, "d": 2, "q": q, "q_pos": t,
    "keys": [list(k) for k, _ in keys], "key_pos": [p for _, p in keys],
    "values": [list(v) for v in values],
    "expected_scores": scores, "expected_prob": prob,
    "expected_out": out, "expected_lse": m + math.log(z),
}
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "rope_d2_closed_form.json"), "w") as f:
    json.dump(doc, f, indent=1)
