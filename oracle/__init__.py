"""CPU oracle for grouped-query attention over a preallocated KV cache.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package. The HIP library never calls it and it never calls the HIP library:
the two share no code, headers, helpers or constants.

Everything is plain numpy in float64, slow on purpose, written so a reader can
check it against the pages by eye:

  * ``direct``     -- the cache (append / truncate / reset / bytes) and the
                      "direct reference" attention: KV heads repeated, a loop
                      over every query, a plain softmax over keys 0..pos.
  * ``vectorised`` -- a second formulation, per (row, KV head) block over
                      the row's own prefix, with the bottom-right triangle
                      as the mask and a log-sum-exp normalisation, used to
                      cross-check ``direct``.
  * ``window``     -- sliding-window attention over a ring-buffer cache whose
                      slots store the absolute positions they hold.
  * ``fp8``        -- an E4M3 cache with one scale per KV head: the format's
                      decoder and round-to-nearest-even encoder, attention on
                      the dequantized values.
  * ``tree``       -- tree-based speculative verify: each draft node attends
                      the committed keys and its ancestors (parent pointers).
  * ``paged``      -- a pool of fixed-size pages shared by all rows and a block
                      table per row; attention over the keys gathered through it.

Where the pages are silent or disagree, the reading taken is stated in the
docstring of the function that depends on it.
"""

from . import direct, fp8, paged, tree, vectorised, window  # noqa: F401
