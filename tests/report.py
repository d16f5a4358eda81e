"""Parity statistics collected by the GPU tests and printed in pytest's terminal summary
(so that a quiet run, -q, still shows each case's token count, near ties and error)."""
LINES = []


def add(line: str) -> None:
    LINES.append(line)
