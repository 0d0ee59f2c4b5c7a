"""Plain CPU oracle for the DFlash gamma-block drafter (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may import this
package. The product path never does.
"""
from .dflash_oracle import *  # noqa: F401,F403
from .dflash_oracle import Drafter, Engine, PagePool, PoolError  # noqa: F401
