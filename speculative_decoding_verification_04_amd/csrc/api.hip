// Host-only entry points of the library.
#include "spec_verify.h"

extern "C" const char *spec_strerror(int code) {
  switch (code) {
    case SPEC_OK: return "ok";
    case SPEC_EINVAL: return "invalid argument";
    case SPEC_EWORKSPACE: return "workspace too small or misaligned";
    case SPEC_ECAPACITY: return "size exceeds a documented maximum";
    case SPEC_EHIP: return "HIP runtime error at launch";
    default: return "unknown error";
  }
}
