"""MI355X-native DSA hot path: lightning-indexer scores, exact top-k and sparse
absorbed-MLA attention over kept latent rows, as hand-written HIP kernels for
gfx950 behind a C ABI (include/dsa.h).  This package holds the thin ctypes
binding (binding.py), the build step (build.py), device upload helpers
(device.py) and the seeded input generator (inputs.py)."""
from .binding import (DsaCache, DsaError, DeviceCache, dsa_cache_append, dsa_decode_shared,
                      dsa_decode_shared_workspace_size, dsa_decode_step, dsa_decode_step_noalloc,  # noqa: F401
                      dsa_decode_step_workspace_size,
                      dsa_decode_window, dsa_decode_window_workspace_size, dsa_index_scores, dsa_status_string, dsa_topk, dsa_topk_workspace_size, dsa_workspace_clear,
                      load, mla_absorb_out, mla_absorb_q, mla_sparse_attend, mla_sparse_attend_workspace_size)
