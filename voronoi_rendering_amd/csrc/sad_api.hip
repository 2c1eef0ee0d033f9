// sad_api.hip -- version and status names of the C ABI.
#include "sad.h"

extern "C" int sad_abi_version(void) { return SAD_ABI_VERSION; }

extern "C" const char* sad_status_string(int status) {
    switch (status) {
        case SAD_OK:
            return "SAD_OK";
        case SAD_EINVAL:
            return "SAD_EINVAL: invalid argument (size, NULL or misaligned pointer, limit, aliasing)";
        case SAD_EUNSUPPORTED:
            return "SAD_EUNSUPPORTED: parameter outside what this library implements";
        case SAD_EHIP:
            return "SAD_EHIP: the HIP runtime refused the launch";
        default:
            return "unknown SAD status";
    }
}
