"""Parity margins measured by the GPU tests, printed in the session summary
(so they appear in the tail of a quiet `pytest -q` run)."""
RECORDS = []


def record(name: str, err: float, tol: float) -> None:
    RECORDS.append((name, float(err), float(tol)))
