"""CPU oracle of the per-frame hot path: 3D rotary embedding, dual-stream paged
KV cache bookkeeping, and attention over the retained tokens.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``rope_paged_kv_amd``) never imports, calls or links anything here, and this
package never imports the product path.  The only module both sides use is
``rpkv_inputs`` (seeded inputs and workload shapes, no arithmetic of the method).

Everything is plain numpy in float64, written from the pages' description:

* ``rope3d``    - per-axis 1D frequency tables, the t/h/w concatenation and the
                  complex rotation of Q and K
                  (page "How 3D RoPE Positional Encoding Works with the Paged KV
                  Cache in LingBot-Map", sections "Multi-Axis Frequency
                  Generation" and "Complex-Valued Tensor Application";
                  page "Video RoPE Positional Encoding: 3D Rotary Embeddings for
                  Long-Sequence Video", sections "The Three Rotary Dimensions" and
                  "NTK-Aware Frequency Scaling").
* ``retained``  - the set of tokens a frame attends to, enumerated directly
                  from the policy (scale frames, sliding window, append-only
                  special stream, keyframes / skip-append), independent of pages.
* ``pages``     - a page-level simulator of the dual-stream cache (free list,
                  scale pages, window, special pages, visible page table,
                  last-page length) used to pin device bookkeeping bit-exactly.
* ``attention`` - dense softmax attention over an explicit key set, with the
                  log-sum-exp.
* ``stream``    - drives the above over a workload, frame by frame.
* ``chain``     - the full-depth chain (QKV projection, alternating frame and
                  cached layers, residual).

Where the pages are silent or contradict each other, the reading taken is
stated at the point of use.  Storage rounding: for bf16 workloads the rotated
Q and the cached K/V are held in bf16 (the cache of the pages' example is
created with dtype bfloat16), so the oracle rounds rotated Q and K to bf16
(nearest, ties to even) before attention; everything else is float64.
"""
