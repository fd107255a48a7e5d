"""Confidence head with sequential temperature scaling -- oracle side (test infrastructure).

Follows the DSpark study notes (pages.layerx.co.jp), section 5.1 "Confidence
Head": for every draft position k the head outputs a scalar, the probability
that the token there survives verification given that all earlier drafts were
accepted, from a light linear projection of the draft's hidden state followed
by a sigmoid. The SGLang article (winzheng.jp) adds Sequential Temperature
Scaling (STS), which calibrates these confidences so that the survival
probability (their running product) tracks the measured acceptance rate.

Readings (the formulas are stripped from the extracted text): the projection
is a dot product with one weight vector w plus a bias b; STS divides the
position's logit by a temperature T_k of that position before the sigmoid
("sequential" = one temperature per draft position), T_k = 1 when no scaling is
given:  c_{i,k} = sigmoid((w . h_{i,k} + b) / T_k), computed in fp64 here.

Pinned by: a unit weight vector picks one hidden coordinate (closed form
sigmoid((h_j + b) / T)); a zero logit gives exactly 1/2; the head is monotone
in the logit and tends to 1/2 as T grows; symmetry sigmoid(-x) = 1 - sigmoid(x)
(tests/test_oracle_confidence.py).
"""
import numpy as np


def confidence_head(h, w, b, temps=None):
    """h [R, K, H] hidden states, w [H], scalar b, temps [K] or None -> conf [R, K] fp64."""
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    logit = h @ w + float(b)
    if temps is not None:
        logit = logit / np.asarray(temps, dtype=np.float64)[None, :]
    return 1.0 / (1.0 + np.exp(-logit))
