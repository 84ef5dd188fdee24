"""Mamba-2 SSM core on MI355X (gfx950): conv1d + chunked SSD scan + in-place decode state update."""
from .configs import Dims, NEMOTRON_H_8B, TINY, WORKLOADS  # noqa: F401
