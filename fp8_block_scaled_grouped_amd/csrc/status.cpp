// Status text for libmoe355.
#include "../../include/moe355.h"

extern "C" const char* moe355_strerror(int status) {
  switch (status) {
    case MOE355_OK: return "moe355: success";
    case MOE355_EINVAL: return "moe355: invalid argument (null pointer, negative size, stride below width or workspace too small)";
    case MOE355_EUNSUPPORTED: return "moe355: unsupported shape or option";
    case MOE355_EMISALIGNED: return "moe355: pointer or row stride not 16-byte aligned";
    case MOE355_ELAUNCH: return "moe355: kernel launch failed";
    case MOE355_ESCRATCH:
      return "moe355: the call needs more device scratch than the library's static scratch array holds";
    default: return "moe355: unknown status";
  }
}
