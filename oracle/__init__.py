"""CPU reference (test infrastructure only): see ``oracle.paged_attention``."""
from . import paged_attention  # noqa: F401
