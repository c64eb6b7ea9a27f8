// k_copy.hip -- placeholder translation unit for device-side copy kernels.
#include "tls_dev.h"
