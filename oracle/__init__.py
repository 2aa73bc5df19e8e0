"""CPU oracle for the Fast-dLLM decoding hot path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute anything in this package: it is used by the tests, by the package's
smoke check and by the benchmark's CPU-baseline leg, and by the committed
script that writes stored expected values. It shares no code with the HIP
path.

It is a plain, slow, float64 implementation of what the method computes,
written from these pages:

* "Fast-dLLM: Training-free Acceleration of Diffusion LLM by Enabling KV
  Cache and Parallel Decoding" -- the paper-graph-ui commentary page
  (cited below as [commentary], with its section numbers), and
* the NVlabs/Fast-dLLM GitHub README (cited as [README]).

Modules:

* ``model``   -- the bidirectional masked-diffusion transformer forward, full
                 and with a block-wise approximate KV cache (PrefixCache or
                 DualCache).
* ``decode``  -- confidence scores, threshold and factor selection with the
                 progress guarantee, and the block-wise decoding loop.
* ``theorem`` -- joint vs product-of-marginals greedy decoding (Theorem 1).

Readings of the pages where they are silent or ambiguous are listed in each
function's docstring. Parity status: every function here is pinned by a
``-m "not gpu"`` test except the approximation error of the cache itself
(cached vs uncached logits of a random model), which is "parity unpinned":
the pages print that quantity only for trained weights.
"""
