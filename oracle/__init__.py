"""Plain CPU oracle of block-sparse attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP library; the only module both sides use is ``synth`` (seeded inputs,
none of the method's arithmetic).

What it follows (the pages are Korean summaries; facts restated, not quoted):

* ``select``  -- the Intra-Block Clustering Selector of the AB-Attention page
  (onedev.kr/papers/1521, section "무엇과 다른가"): 128-query blocks, 4-token
  KV blocks, one k-means iteration with 8 clusters inside each query block,
  block score = cluster-share-weighted softmax mass of the centroids over the
  pooled keys.
* ``plan``    -- SIP of the same page (section "어떻게 쓰나"): inclusion
  probabilities pi = min(1, lambda * S) summing to the budget s, systematic
  sampling of exactly s distinct blocks shared by the query block; and top-k
  at the same budget (section "무엇과 다른가" premise; the ablation paragraph
  of "전제와 한계" equates SIP without pi weighting with top-k).
* ``attn``    -- the fused pass of the same page (section "전제와 한계",
  first paragraph): softmax over the gathered keys with logits shifted by
  -log pi, written as the plain definition (gather, one dense softmax).
* ``basa``    -- BASA page (onedev.kr/papers/688): shifted windows spanning
  all frames, pooled K/V memory, routed raw windows; key set = own window
  U routed windows U pooled memory.
* ``diag``    -- accuracy diagnostics of a plan (AB-Attention page, sections
  "무엇과 다른가", "어떻게 쓰나" and the ablation paragraph of "전제와 한계"):
  the true attention mass of every KV block per query block, the mass a
  plan retains, the oracle top-k by that mass, and the output error against
  dense attention.

Precision: fp64 everywhere, with one deliberate exception.  The k-means
assignment (an argmin) and the BASA window routing (a top-2) are discrete
decisions taken from floating-point values; both sides take them in fp32 in
one stated operation order (sequential sums, no fused multiply-add, IEEE
division), so that the same decision is reached.  Everything downstream of
those decisions is fp64 again.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, special cases, brute force or figures printed on the
pages.  The pages' quality claims (dB, retained mass, 41 % lower error) were
measured on real model activations; ``diag`` computes the same quantities on
the seeded synthetic inputs, whose values are not expected to match the
pages' figures.
"""

from . import splitmix, select, plan, attn, basa, diag  # noqa: F401
