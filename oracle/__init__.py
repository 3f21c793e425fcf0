"""CPU oracle of mla_post (test infrastructure only; see ``oracle.post``)."""
from .post import *  # noqa: F401,F403
from .post import __all__  # noqa: F401
