"""CPU oracle for one Hydra/Medusa draft-and-verify round.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product
package never imports it, and it imports nothing from the product package.
"""
from .hydra_oracle import *  # noqa: F401,F403
