"""CPU oracle for DSA select + attend and block-sparse MSA. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package. The product path (``sparse_attention_dsa_amd``) never imports it, and this
package imports nothing from the product path.
"""
from .dsa_oracle import *  # noqa: F401,F403
from . import msa_oracle  # noqa: F401
