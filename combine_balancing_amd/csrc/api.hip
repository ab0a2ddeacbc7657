// Status strings and version of the mep C ABI.
#include "mep.h"

extern "C" const char* mep_status_str(int status) {
    switch (status) {
        case MEP_OK: return "MEP_OK";
        case MEP_ERR_NULLPTR: return "MEP_ERR_NULLPTR: a required pointer is NULL";
        case MEP_ERR_PARAM: return "MEP_ERR_PARAM: invalid parameter value or combination";
        case MEP_ERR_SHAPE: return "MEP_ERR_SHAPE: size out of range or misaligned row pointer";
        case MEP_ERR_HIP: return "MEP_ERR_HIP: HIP runtime error at launch";
        default: return "unknown mep status";
    }
}

extern "C" int mep_version(void) { return 100; }
