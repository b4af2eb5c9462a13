// The dense chain with a transformed draft (T != 1, no top-k): final draw from
// precomputed row statistics, one workgroup of 512 threads per batch row; the
// implementation is dense_impl.hpp.
#define SV_DENSE_THREADS 512
#define SV_DENSE_WALK 0
#define SV_DENSE_TR 1
#include "dense_impl.hpp"
