"""CPU oracle for range-masked attention (test infrastructure only; the library never imports it)."""
from .ffa_oracle import (FULL, CAUSAL, normalise_slices, slice_cells, visibility, visible_count,
                         attention_fwd, attention_bwd, tile_set)
