"""Writes worked_example.json: a constructed worked example of the online
softmax recurrence, derived by hand-sized arithmetic with Python's ``math``.

The page "FlashAttention: making attention IO-aware" ("Online softmax") says a
figure runs the recurrence on real numbers, but that figure did not survive in
the page text, so this example is constructed instead.  One query row, head
dimension 1, scale 1, key tiles of two columns:

    scores  s = [1, 3 | 2, 5]   (q = 1, k = [1, 3, 2, 5])
    values  v = [1, 2, 3, 4]

Two-pass softmax:  m = 5, l = e^-4 + e^-2 + e^-3 + e^0, P_k = e^(s_k - 5) / l,
O = sum_k P_k v_k, L = m + ln l.
Online, tile 1 (s = 1, 3): m = 3, correction = 0 (m started at -inf),
l = e^-2 + 1, acc = 1 e^-2 + 2.
Online, tile 2 (s = 2, 5): m = 5, correction = e^-2,
l = (e^-2 + 1) e^-2 + e^-3 + 1, acc = (e^-2 + 2) e^-2 + 3 e^-3 + 4.
Backward row term with dO = 0.5:  D = dO * O.

This script uses only ``math``; it calls neither the oracle nor the GPU path.
"""
import json
import math
import os

s = [1.0, 3.0, 2.0, 5.0]
v = [1.0, 2.0, 3.0, 4.0]
m = 5.0
e = [math.exp(x - m) for x in s]
l = math.fsum(e)
P = [x / l for x in e]
O = math.fsum(p * vv for p, vv in zip(P, v))
L = m + math.log(l)
t1_m = 3.0
t1_l = math.exp(1.0 - 3.0) + math.exp(0.0)
t1_acc = 1.0 * math.exp(-2.0) + 2.0 * 1.0
corr2 = math.exp(3.0 - 5.0)
t2_l = t1_l * corr2 + math.exp(2.0 - 5.0) + math.exp(0.0)
t2_acc = t1_acc * corr2 + 3.0 * math.exp(-3.0) + 4.0
fixture = {
    "source": "constructed; the page's own numeric figure for the online "
              "softmax is missing from its text (FlashAttention: making "
              "attention IO-aware, 'Online softmax')",
    "q": [[1.0]], "k": [[x] for x in s], "v": [[x] for x in v],
    "scale": 1.0, "Br": 1, "Bc": 2,
    "two_pass": {"m": m, "l": l, "P": P, "O": O, "L": L},
    "online": [
        {"tile": 0, "m": t1_m, "correction": 0.0, "l": t1_l, "acc": t1_acc},
        {"tile": 1, "m": 5.0, "correction": corr2, "l": t2_l, "acc": t2_acc},
    ],
    "backward": {"dO": 0.5, "D": 0.5 * O},
}
out = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                   "worked_example.json")
with open(out, "w") as f:
    json.dump(fixture, f, indent=1)
    f.write("\n")
print(json.dumps(fixture["two_pass"]), json.dumps(fixture["online"]))
