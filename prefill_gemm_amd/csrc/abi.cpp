// Status strings and version of libpg.
#include "pg.h"

extern "C" const char *pg_strerror(int code) {
    switch (code) {
        case PG_OK: return "ok";
        case PG_EINVAL: return "invalid argument (null pointer, non-positive size, misalignment or aliasing)";
        case PG_EUNSUPPORTED: return "shape not supported by the kernels (nothing enqueued)";
        case PG_ELAUNCH: return "kernel launch failed";
        case PG_EWORKSPACE: return "workspace missing or too small";
        case PG_ETIMEOUT: return "a device-wide barrier wait gave up: the frame outputs since the workspace was set up are not trustworthy";
        default: return "unknown status";
    }
}

extern "C" const char *pg_version(void) { return "0.1.0 gfx950"; }
