"""CPU oracle (float64) for exact varlen attention. Test infrastructure only.

Only the tests, the smoke check and the bench's CPU-baseline leg import this
package; the product path never does.
"""
from .attention import *  # noqa: F401,F403
from .attention import __all__  # noqa: F401
