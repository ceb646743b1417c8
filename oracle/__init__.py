"""CPU oracle for the tree-verify attention and the partial-KV-cache step.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The product path (the
HIP library and its Python binding) never imports, calls or links it, and this
package imports nothing from the product path.

Everything here is plain numpy in float64: the plain definitions of what the
fast path computes, with no blocking, splitting or fusion. bf16 inputs arrive
as uint16 bit patterns and are widened exactly to float64 here.

Functions and the passages they follow (TokenSwift pages):

* ``ancestor_mask``      the tree mask over draft tokens (tool listing, "How it
                          works": candidates are organised as a tree and
                          attend along it).
* ``verify_attn_ref``     masked softmax attention of the draft queries over
                          the whole cache plus their own ancestors (tool
                          listing, "How it works": the target model checks all
                          drafts in one pass against its complete cache).
* ``draft_attn_ref``      the same over the gathered partial cache with a
                          causal chain of new tokens (tool listing, "How it
                          works": drafting runs the target model itself on a
                          reduced cache).
* ``importance_ref``      query-key importance per chunk (summary page,
                          "Approach": the reduced cache is re-selected by how
                          strongly queries attend to its keys).
* ``topk_ref``            the highest-scoring chunks up to the budget
                          (model card CLI example: retrieval budget 4096).
* ``gather_ref``          the partial cache built from the chosen chunks.
* ``accept_ref``          the longest valid draft path, one picked at random
                          among equals (tool listing, "How it works": drafts
                          are checked for an exact match with the target's
                          tokens and one of the longest is chosen at random).
* ``commit_ref``          the KV cache updated with the accepted drafts (same
                          passage).
* ``build_tree_ref``      the candidate tree from the per-position logits
                          (tool listing, "How it works"; tree shapes from the
                          summary page's ablation table).
* ``sample_ref``          the target's token per verified position: windowed
                          repetition penalty, temperature, min-p, and a draw
                          from the caller's uniform (model card CLI example;
                          summary page, "Approach" and ablation table).
* ``ngram_table``, ``ngram_update``, ``retrieve_ref``  the 4-gram table of the
                          committed text and the top-k 4-grams for a first
                          token (tool listing, "How it works"; model card CLI
                          example: top-k 20).

Pinned by ``tests/test_oracle_*.py`` (brute force in 50-digit arithmetic,
reductions to torch's scaled-dot-product attention, closed forms, a rank-count
definition of top-k, hand-worked examples, scipy's softmax for the sampler). The importance reduction order (max over the grouped
heads, mean over tokens and recent queries) is a reading of the pages: the
pages name query-key importance but not the reduction, so that choice is
pinned only by its own definition.
"""
from .attention import ancestor_mask, verify_attn_ref, draft_attn_ref, widen
from .partial_kv import importance_ref, topk_ref, gather_ref
from .accept import accept_ref, commit_ref
from .tree import build_tree_ref
from .sample import sample_ref
from .ngram import ngram_table, ngram_update, retrieve_ref

__all__ = ["ancestor_mask", "verify_attn_ref", "draft_attn_ref", "widen",
           "importance_ref", "topk_ref", "gather_ref", "accept_ref", "commit_ref",
           "build_tree_ref", "sample_ref", "ngram_table", "ngram_update", "retrieve_ref"]
