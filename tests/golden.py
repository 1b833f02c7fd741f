"""Readers for the text fixtures under tests/golden (values printed on the pages)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


class Printed(float):
    """A number as printed on a page; ``tol`` is half a unit of its last printed digit."""

    def __new__(cls, text: str):
        obj = super().__new__(cls, float(text))
        decimals = len(text.split(".")[1]) if "." in text else 0
        obj.tol = 0.5 * 10.0 ** (-decimals)
        return obj


def keyed(name):
    """'key v1 v2 ...' lines -> {key: [Printed]}."""
    return {parts[0]: [Printed(x) for x in parts[1:]] for parts in _lines(name)}


def rows(name):
    """Whitespace-separated integer rows."""
    return [[int(x) for x in parts] for parts in _lines(name)]
