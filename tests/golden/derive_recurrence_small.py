"""Recompute the exact results in recurrence_small.txt with rational arithmetic.

Independent of the oracle: it applies the matrix form of the update from
"Decoding Hybrid Linear Attention Architectures", sec. 3, item 6,
M <- (I - beta k k^T) Diag(alpha) M + beta k v^T, o = M^T q, with
fractions.Fraction entries.  Run as a script it checks the fixture file.
"""
from fractions import Fraction
import os


def parse_matrix(text):
    return [[Fraction(x.strip()) for x in row.split(",")] for row in text.split(";")]


def read_cases(path):
    cases, cur = {}, None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("[case"):
            cur = line[len("[case"):].strip(" ]")
            cases[cur] = {}
            continue
        key, val = line.split(":", 1)
        cases[cur][key.strip()] = val.strip() if key.strip() == "gate" else parse_matrix(val)
    return cases


def run_exact(case):
    M = [row[:] for row in case["M0"]]
    dk, dv = len(M), len(M[0])
    outs = []
    for t in range(len(case["k"])):
        k, v, q = case["k"][t], case["v"][t], case["q"][t]
        beta = case["beta"][t][0]
        alpha = case["alpha"][t]
        a = [alpha[0]] * dk if len(alpha) == 1 else alpha
        D = [[a[i] * M[i][j] for j in range(dv)] for i in range(dk)]          # Diag(alpha) M
        E = [[(1 if i == l else 0) - beta * k[i] * k[l] for l in range(dk)] for i in range(dk)]
        M = [[sum(E[i][l] * D[l][j] for l in range(dk)) + beta * k[i] * v[j]
              for j in range(dv)] for i in range(dk)]
        outs.append([sum(M[i][j] * q[i] for i in range(dk)) for j in range(dv)])
    return outs, M


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "recurrence_small.txt")
    for name, case in read_cases(path).items():
        o, M = run_exact(case)
        assert o == case["o"], (name, o)
        assert M == case["MT"], (name, M)
        print(name, "ok")
