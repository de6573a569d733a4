"""Error figures of the headline parity cases, collected during a test run
and printed in pytest's terminal summary (so they show under -q too)."""

LINES = []


def record(line):
    LINES.append(line)
