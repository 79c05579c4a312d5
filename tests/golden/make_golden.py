"""Writes tests/golden/special_values.json from the oracle's scalar singular-value map.

The values are closed forms: one NS step multiplies every singular value sigma of
the short-side tile by the polynomial a + b sigma^2 + c sigma^4, so K steps send
sigma to phi^K(sigma) with phi(x) = a x + b x^3 + c x^5 (a polynomial matrix
function acts on the spectrum; Higham, Functions of Matrices, 2008, cited by
"SignMuon: Communication-Efficient Distributed Muon Optimization", References).
They can be checked with a pocket calculator; the tests compare the matrix
iteration of the oracle (and of the GPU path) against them.

Run:  python tests/golden/make_golden.py
"""
import json
import math
import os
import sys

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "..", ".."))
import oracle  # noqa: E402

Q = oracle.COEFFS_QUINTIC
C = oracle.COEFFS_CUBIC

cases = []
for name, co in (("quintic", Q), ("cubic", C)):
    for K in (1, 2, 5, 8):
        cases.append({"what": "rank-1 tile: normalised tile has one singular value 1",
                      "coeffs": name, "K": K, "x0": 1.0, "value": oracle.phi_iterate(1.0, K, co)})
    for T in (32, 64, 128):
        cases.append({"what": f"{T}x{T} orthogonal tile: all {T} singular values are 1/sqrt({T})",
                      "coeffs": name, "K": 5, "x0": 1.0 / math.sqrt(T),
                      "value": oracle.phi_iterate(1.0 / math.sqrt(T), 5, co)})

doc = {
    "source": "closed form phi^K(x0), phi(x) = a x + b x^3 + c x^5; "
              "coefficient sets cubic (1.5, -0.5, 0) and quintic (3.4445, -4.7750, 2.0315)",
    "written_by": "tests/golden/make_golden.py (calls oracle.phi_iterate only)",
    "cases": cases,
}
path = os.path.join(os.path.dirname(__file__), "special_values.json")
with open(path, "w") as f:
    json.dump(doc, f, indent=1)
print("wrote", path, len(cases), "cases")
