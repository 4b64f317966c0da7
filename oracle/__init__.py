"""CPU oracle for token-pruned self-attention with a persistent KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or calls
this package: only the tests, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP library (no kernels, headers, helpers
or constant tables); the only thing both sides share is the seeded input
generator in ``workloads``, which holds none of the method's arithmetic.

``reference`` is the plain numpy float64 implementation of every step;
``brute`` is a second, independent pure-Python implementation used to pin the
first on tiny inputs.

Sources (cited by page title and section; the pages are gist.science
summaries of the papers):

* HSA -- "Resumen Técnico: Asignación de Pasos Heterogénea (HSA) para la
  Generación Eficiente de Video" (gist.science/es/paper/2605.06892):
  §2.1 token partition and schedule, §2.2 KV-cache synchronisation,
  §2.3 cached Euler update, §2.4 phase-aware cache window.
* LIPAR -- "Training-free Latent Inter-Frame Pruning with Attention Recovery"
  (gist.science/es/paper/2603.05811 and gist.science/nl/paper/2603.05811):
  §2.B latent inter-frame pruning (with its short- and long-term change
  mask), §2.C attention recovery (noise-aware duplication), Dutch §2.D
  restoration.

Parity status of each function is stated in its docstring; the end-to-end
layer is pinned only through its pinned steps (there is no worked example on
any page).
"""

from . import brute, reference

__all__ = ["reference", "brute"]
