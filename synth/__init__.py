"""Seeded synthetic inputs (shared by the tests, the smoke check and the
benchmark).  Holds no arithmetic of the method: draws and storage casts only."""
from . import configs, gen

__all__ = ["configs", "gen"]
