// The dense chain (T == 1, no top-k) as one walk per batch row, one workgroup
// of 512 threads each; the implementation is dense_impl.hpp.
#define SV_DENSE_THREADS 512
#define SV_DENSE_WALK 1
#define SV_DENSE_TR 0
#include "dense_impl.hpp"
