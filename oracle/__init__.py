"""CPU oracle for the LSA layer hot path.

TEST INFRASTRUCTURE ONLY.  Plain NumPy in float64, slow and written to be read
against the method description (zhichai.net explainer, ch.2 "semantic
clustering", ch.3 "query path", ch.4 "tree"; diosapp.com.cn tutorial, section
二, pseudocode).  Only the tests, the smoke check and the CPU-baseline leg of
the benchmark may import it; the library never does, and it shares no code
with the HIP path.
"""

from .lsa_oracle import *  # noqa: F401,F403
from .lsa_oracle import __all__  # noqa: F401
