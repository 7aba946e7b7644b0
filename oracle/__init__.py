"""fp64 CPU oracle for exact attention (test infrastructure; see attention.py's header)."""
