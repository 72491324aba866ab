// Gated low-rank delta of R-ISD (isd_lora_delta): see isd.h.
#include "device_common.hpp"
#include "isd_internal.hpp"
