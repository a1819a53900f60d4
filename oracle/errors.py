"""Error kinds of the oracle (test infrastructure).

The kinds are the variants of ``SparseAttentionError`` on the types.rs page
(alice-llm 2.0.0, ``SparseAttentionError``). The oracle raises them with the
same ``what`` / ``expected`` / ``got`` detail that the page's variants carry.
"""


class SparseAttentionError(Exception):
    """One of: HeadCountMismatch, BlockPageMismatch, CuSeqlensInvalid,
    ShapeMismatch, SelectedOutOfRange, HeadDimMismatch, EmptyInput."""

    def __init__(self, kind, what=None, expected=None, got=None):
        self.kind = kind
        self.what = what
        self.expected = expected
        self.got = got
        super().__init__(f"{kind}(what={what!r}, expected={expected}, got={got})")
