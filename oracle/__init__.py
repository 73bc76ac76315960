"""Oracle package (test infrastructure only; see onebit.py's header)."""
