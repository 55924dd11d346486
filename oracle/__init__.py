"""Plain CPU oracle of the HTTM layer (test infrastructure only; see httm_oracle)."""
from .httm_oracle import *  # noqa: F401,F403
from .httm_oracle import Params  # noqa: F401
