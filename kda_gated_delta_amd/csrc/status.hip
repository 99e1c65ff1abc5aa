// Status strings of the C ABI.
#include "kda_host.h"

extern "C" const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
    case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE: a size is out of range or inconsistent";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: K and V must be 128";
    case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN: a pointer or stride is not 16-byte aligned";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: the HIP runtime reported a launch error";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
    default: return "unknown kda_status";
  }
}

// Hash of the sources and flags this library was compiled from (the build
// passes it in); lets a caller check that a loaded binary matches a source
// tree.
#ifndef KDA_SOURCE_HASH
#error "build with -DKDA_SOURCE_HASH=... (see build.py)"
#endif
extern "C" const char* kda_build_id(void) { return KDA_SOURCE_HASH; }
