"""Loader for the worked examples under tests/golden/."""
import json
import os

_HERE = os.path.dirname(os.path.abspath(__file__))


def golden(name: str):
    with open(os.path.join(_HERE, "golden", "worked_examples.json")) as f:
        return json.load(f)[name]
