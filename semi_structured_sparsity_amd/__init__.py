"""MI355X-native N:M semi-structured sparsity: importance scores, top-N group
masks, packing, the (2N-2):2N sliding-window decomposition, Hutchinson and
soft-gate mask annealing, and the structured-sparse linear layer on gfx950
SMFMAC.  The compute lives in libnmsparse.so (C ABI: include/nmsparse.h);
this package is its ctypes binding."""
from ._binding import *  # noqa: F401,F403
from ._binding import (NMError, raw, last_error, lifted_width, index_words, LIB_PATH,  # noqa: F401
                       NM_F32, NM_BF16, NM_I8, NM_I32, NM_SCORE_HESSIAN, NM_SCORE_MAGNITUDE)
