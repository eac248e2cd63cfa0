"""fp64 CPU oracle for paged MLA decode (test infrastructure only)."""
