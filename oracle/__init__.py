"""CPU oracle of the KDA token mixer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the HIP
library and its Python binding) never imports, links or calls it, and shares no
code with it.

Two independent implementations live here:

* ``kda_oracle.c`` -- plain C, fp64, OpenMP over (sequence, head); the
  token-by-token definition.  Wrapped by :mod:`oracle.c_oracle`.
* ``kda_ref.py``   -- NumPy fp64: the same definitions, plus the chunkwise form
  and a brute-force dense-transition form used to pin the recurrence.

Pages cited (by title and panel):

* "Inside Kimi K3" (lei.chat): the Kimi Delta Attention one-head diagram and
  the KDA short-convolution diagram.
* "Animated Kimi K3 architecture diagram" (github.io): the local-memory panel
  and its notebook trace.
"""
