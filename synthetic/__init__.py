"""Seeded synthetic workloads: shapes of the five benchmark configurations and
the input recipes.  Holds none of the attention method's arithmetic; both the
GPU path's tests/bench and the CPU oracle's tests draw their inputs here."""
from .configs import C5_FRACS, CONFIGS, Config, c5_variant, get_config  # noqa: F401
from .inputs import make_inputs  # noqa: F401
