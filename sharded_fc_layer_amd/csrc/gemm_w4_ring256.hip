// Ring-kernel instances with 256-column block tiles (see gemm_w4_ring_impl.h).
#define FCW4_RING_BN 256
#include "gemm_w4_ring_impl.h"
