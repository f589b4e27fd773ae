"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark."""
from .inputs import *  # noqa: F401,F403
