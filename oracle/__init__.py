"""fp64 CPU oracle (test infrastructure only; the library never imports it)."""
from .tree_oracle import (GDN, SCALAR_DECAY, STATUS_OK, STATUS_BAD_PARENTS,  # noqa: F401
                          STATUS_BAD_ACCEPTED, parents_valid, node_path, tree_index,
                          accepted_paths, gdn_step, scalar_step, verify_head, verify,
                          commit_head, commit)
