"""Max err/bound of every parity comparison in this test session.

Tests call record(); tests/conftest.py prints the table at the end of the
session (also under -q, where pytest hides what passing tests print), so
that a run's log shows how close each case came to the bound."""
RATIOS: list[tuple[str, float]] = []
NOTES: list[str] = []


def record(name: str, ratio: float) -> None:
    RATIOS.append((name, float(ratio)))


def note(text: str) -> None:
    """A line printed with the table (measurements that are not ratios)."""
    NOTES.append(text)
