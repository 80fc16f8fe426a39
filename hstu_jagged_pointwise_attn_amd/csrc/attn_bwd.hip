// Backward attention kernels (filled in with the backward pass).
#include "hstu_internal.h"
