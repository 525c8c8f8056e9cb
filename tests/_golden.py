"""Readers for the text fixtures under tests/golden (comment lines start with '#')."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.strip()
            if ln and not ln.startswith("#"):
                yield ln


def table(name, sep="|"):
    return [[c.strip() for c in ln.split(sep)] for ln in lines(name)]
