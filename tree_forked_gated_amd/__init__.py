"""Tree-structured gated delta rule on MI355X (gfx950).

``tree_forked_gated_amd.binding`` wraps the C ABI of ``libgdn_tree.so``
(include/gdn_tree.h) and raises on import if the library is not built;
``tree_forked_gated_amd.workloads`` draws seeded synthetic tree streams and
needs no GPU build.
"""
