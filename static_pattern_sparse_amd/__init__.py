"""Fibonacci-spaced sparse attention for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libfsa.so`` (hand-written HIP kernels);
``static_pattern_sparse_amd.fsa`` is its thin Python binding. Importing this
package loads nothing; the library is opened on the first binding call and a
missing library raises at that point.
"""
